/*
 * ep_oracle.c — plain, slow CPU oracle for MoE expert-parallel dispatch and
 * combine on one GPU's share of an EP group.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header, table or helper with the HIP library; it is built with
 * -O2 -fno-fast-math -ffp-contract=off so that no contraction or reassociation
 * changes the arithmetic written here.
 *
 * Sources (cited by page and section; the pages are the text of three web
 * pages on GPU-initiated EP communication):
 *   [UCCL]  UCCL-EP article, peacm.com/news/835744
 *           s2.1 architecture (GPU writes TransferCmd into a local FIFO),
 *           s2.2 FIFO details (RingBuffer, batches of up to 8, 256 in flight),
 *           s2.3 proxy loop (PostRDMAWrite(dst_rank, src_offset, dst_offset,
 *           size)), s3.1 the four message types, s3.2 op/value encoding
 *           (4-bit op, 28-bit value), s4.1 LL token packing ("small tokens
 *           merged into one message", batch 8), s4.2 HT 8 channels,
 *           s5.2 tuning table (FIFO depth 1024, 256 in flight, 8 channels),
 *           s6 EP32 dispatch/combine measurements.
 *   [GIN]   NCCL GIN article, bjdmk.com.cn/news/2086017, s3.1.1 dynamic
 *           token routing (each token is sent to the owner of its expert).
 *   [NOTES] GPU communication notes, blog.zhenwei.site, s5 optimisation list
 *           (DeepEP dispatch/combine, combine overlapped with the next layer).
 * The pages never print the dispatch/combine arithmetic.  Where they are
 * silent the plainest reading is used; each reading is stated at the place
 * where it is applied.
 *
 * Parity status of each function:
 *   oracle_layout         pinned: brute-force set enumeration, invariants
 *   oracle_pack           pinned: byte equality with x rows, metadata sums
 *   oracle_e4m3_encode    pinned: nearest-code search over all finite codes,
 *                         torch float8_e4m3fn, OCP worked values
 *   oracle_quantize_row   pinned: max code per block, error bound, round trip
 *   oracle_descriptors    pinned: tiling invariants, counts
 *   oracle_combine        pinned: per-expert brute force, identity, scaling
 *   oracle_ll_layout      pinned: brute-force per-expert enumeration, invariants
 *   oracle_ll_pack        pinned: byte equality with x rows per (t, j)
 *   oracle_ll_descriptors pinned: tiling invariants, counts, brute-force grouping
 *   oracle_ll_combine     pinned: per-choice brute force, identity, agreement
 *                         with oracle_combine on identity experts
 *   end-to-end values vs the pages: parity unpinned (no printed example)
 *
 * Threads: pack and combine handle each token on its own, so their token
 * loops may be split over OpenMP threads (oracle_set_threads; the CPU
 * baseline times one thread and all host cores).  A token's arithmetic and
 * its order are the same on any number of threads.  Layout and descriptors
 * are sequential by definition (running counters) and stay on one thread.
 */

#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_INVALID_ARG 1
#define ORC_ERR_BAD_EXPERT 2
#define ORC_ERR_CAPACITY 3

#define ORC_FMT_BF16 0
#define ORC_FMT_FP8 1

#define ORC_CMD_WRITE 1
#define ORC_CMD_ATOMIC 2
#define ORC_ATOMIC_ADD 1

/* One transfer command as the proxy would see it.  Field meaning follows the
 * proxy loop of [UCCL] s2.3 (dst_rank, src_offset, dst_offset, size) and the
 * op/value pair of s3.2.  This is the oracle's own record; the byte layout is
 * the interface format both sides agree on (32 bytes). */
typedef struct {
    uint32_t seq;           /* not produced by the oracle: 0 */
    uint8_t type;
    uint8_t op;
    uint16_t num_tokens;
    uint32_t dst_rank;
    uint32_t size_or_value;
    uint64_t src_offset;
    uint64_t dst_offset;
} orc_cmd_t;

/* ---------------------------------------------------------------- helpers */

static float bf16_to_float(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

int64_t oracle_row_bytes(int H, int fmt) {
    if (fmt == ORC_FMT_BF16) return 2LL * H;
    /* reading: H code bytes, then H/128 fp32 scales, then zero bytes up to
     * the next multiple of 128 (the row pitch is a whole number of 128-byte
     * lines) */
    int64_t payload = (int64_t)H + 4LL * (H / 128);
    return (payload + 127) / 128 * 128;
}

/* Threads used by the token loops of pack and combine (n >= 1); returns the
 * number in effect (1 when built without OpenMP). */
int oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ------------------------------------------------------------ routing layout
 * Rank membership, histograms, offsets and stable send slots.
 * Reading: expert e lives on rank e / (E/R) (contiguous blocks of experts).
 * Reading: the unit of dispatch is the (token, destination rank) pair: a token is
 *     sent once to each rank that owns at least one of its top-k experts
 *     ([GIN] s3.1.1 sends each token to the owner of its expert; [UCCL] s1
 *     token-level exchange with dozens of peers).
 * Reading: inside a rank's segment, rows are in ascending token order.
 * Reading: expert id -1 is a dropped choice and is skipped; any other id outside
 *     [0,E) is an error (ORC_ERR_BAD_EXPERT); outputs are then unspecified.
 */
int oracle_layout(int T, int E, int R, int k, const int32_t* topk_idx,
                  int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                  int32_t* rank_offset, int32_t* expert_offset,
                  uint8_t* is_token_in_rank, int32_t* send_slot) {
    if (T < 0 || E < 1 || R < 1 || R > 64 || E % R != 0 || k < 1) return ORC_ERR_INVALID_ARG;
    int epr = E / R;
    for (int r = 0; r < R; r++) num_tokens_per_rank[r] = 0;
    for (int e = 0; e < E; e++) num_tokens_per_expert[e] = 0;
    for (int64_t i = 0; i < (int64_t)T * R; i++) is_token_in_rank[i] = 0;

    /* membership and per-expert histogram */
    for (int t = 0; t < T; t++) {
        for (int j = 0; j < k; j++) {
            int e = topk_idx[(int64_t)t * k + j];
            if (e == -1) continue;
            if (e < -1 || e >= E) return ORC_ERR_BAD_EXPERT;
            num_tokens_per_expert[e] += 1;
            is_token_in_rank[(int64_t)t * R + e / epr] = 1;
        }
    }
    /* per-rank histogram: each token counts once per rank */
    for (int r = 0; r < R; r++)
        for (int t = 0; t < T; t++)
            num_tokens_per_rank[r] += is_token_in_rank[(int64_t)t * R + r];

    /* exclusive scans */
    rank_offset[0] = 0;
    for (int r = 0; r < R; r++) rank_offset[r + 1] = rank_offset[r] + num_tokens_per_rank[r];
    expert_offset[0] = 0;
    for (int e = 0; e < E; e++) expert_offset[e + 1] = expert_offset[e] + num_tokens_per_expert[e];

    /* stable slots: rank-major, ascending token within a rank */
    for (int r = 0; r < R; r++) {
        int32_t c = 0;
        for (int t = 0; t < T; t++) {
            int64_t i = (int64_t)t * R + r;
            if (is_token_in_rank[i]) {
                send_slot[i] = rank_offset[r] + c;
                c++;
            } else {
                send_slot[i] = -1;
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------ fp8 e4m3
 * OCP 8-bit floating point, E4M3 ("FN": no infinities).  Written from the
 * format definition: sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN, so the largest
 * finite magnitude is S.1111.110 = 1.75 * 2^8 = 448.  Conversion from float
 * rounds to nearest, ties to even, and saturates magnitudes beyond 448 to 448
 * (reading: OCP E4M3FN with saturation; the pages never name an fp8 format).
 * The sign bit is kept for zero and for values that round to zero.
 * NaN input gives 0x7F with the input's sign.
 */
uint8_t oracle_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);            /* a = f * 2^e2 with f in [0.5,1): floor(log2 a) = e2-1 */
    int E = e2 - 1;
    if (E < -6) {
        /* subnormal range: quantum 2^-9 */
        double m = nearbyint(ldexp(a, 9));   /* exact scaling, round half to even */
        /* m == 8 is the smallest normal 2^-6, whose code is also 8 */
        return (uint8_t)(sign | (uint8_t)m);
    }
    /* normal: quantum 2^(E-3), mantissa m in [8,16] after rounding */
    double m = nearbyint(ldexp(a, 3 - E));
    if (m == 16.0) { E += 1; m = 8.0; }
    int code = ((E + 7) << 3) | ((int)m - 8);
    if (code > 0x7E) code = 0x7E;   /* rounding up past 448: saturate */
    return (uint8_t)(sign | code);
}

void oracle_e4m3_encode_array(int64_t n, const float* v, uint8_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode(v[i]);
}

float oracle_e4m3_decode(uint8_t c) {
    int s = c >> 7, ex = (c >> 3) & 0xF, man = c & 7;
    double v;
    if (ex == 0xF && man == 7) return NAN;
    if (ex == 0) v = ldexp((double)man, -9);
    else v = ldexp(1.0 + man / 8.0, ex - 7);
    return (float)(s ? -v : v);
}

/* Quantise one bf16 row of H elements into the fp8 row format (reading):
 * H code bytes, then H/128 float32 scales, then zero padding to the row pitch
 * (oracle_row_bytes).  Per 128-element block b (reading):
 *   amax = max |x_i|  (exact in float),  a = max(amax, 1e-4f),
 *   inv = 448 / a  (one IEEE float division),
 *   q_i = e4m3(x_i * inv)  (one IEEE float multiply, then the conversion),
 *   s_b = a / 448  (one IEEE float division).
 * Dequantised value: q_i * s_b.
 * Non-finite inputs (reading; the pages fix no fp8 behaviour): a NaN has no
 * magnitude, so it takes no part in amax; an infinity does, which makes amax
 * and the scale infinite and inv zero.  A product x_i * inv that is NaN (x_i
 * NaN, or x_i infinite with inv = 0) gets the NaN code 0x7F with the sign of
 * x_i, so the sign never depends on how a platform signs a NaN it creates. */
void oracle_quantize_row(int H, const uint16_t* xrow, uint8_t* out_row) {
    int nb = H / 128;
    uint8_t* codes = out_row;
    uint8_t* scales = out_row + H;
    for (int b = 0; b < nb; b++) {
        float amax = 0.0f;
        for (int i = 0; i < 128; i++) {
            float v = fabsf(bf16_to_float(xrow[b * 128 + i]));
            if (v > amax) amax = v;
        }
        float a = amax > 1e-4f ? amax : 1e-4f;
        float inv = 448.0f / a;
        for (int i = 0; i < 128; i++) {
            float xv = bf16_to_float(xrow[b * 128 + i]);
            float prod = xv * inv;
            if (isnan(prod))
                codes[b * 128 + i] = (uint8_t)((signbit(xv) ? 0x80 : 0x00) | 0x7F);
            else
                codes[b * 128 + i] = oracle_e4m3_encode(prod);
        }
        float s = a / 448.0f;
        memcpy(scales + 4 * b, &s, 4);
    }
    int64_t pitch = oracle_row_bytes(H, ORC_FMT_FP8);
    for (int64_t i = (int64_t)H + 4LL * nb; i < pitch; i++) out_row[i] = 0;
}

/* ------------------------------------------------------------ pack
 * For every (t, r) with is_token_in_rank: row t (bf16 bytes, or its fp8 row)
 * goes to send_buf row send_slot[t,r] ([UCCL] s4.1 "prepare token data" before
 * posting the transfer).  Per-slot metadata (reading): slot_src[s] = t;
 * slot_local_idx[s,j] = e_j - r*epr if e_j lives on r else -1;
 * slot_local_w[s,j] = w[t,j] if e_j lives on r else 0.
 * Rows with s >= capacity are not written and ORC_ERR_CAPACITY is returned. */
int oracle_pack(int T, int H, int E, int R, int k, int fmt,
                const uint16_t* x, const int32_t* topk_idx, const float* topk_w,
                const int32_t* send_slot, uint8_t* send_buf, int64_t capacity_rows,
                int32_t* slot_src, int32_t* slot_local_idx, float* slot_local_w) {
    if (E % R != 0) return ORC_ERR_INVALID_ARG;
    if (fmt == ORC_FMT_FP8 && H % 128 != 0) return ORC_ERR_INVALID_ARG;
    int epr = E / R;
    int64_t rb = oracle_row_bytes(H, fmt);
    int status = ORC_OK;
    if (fmt == ORC_FMT_FP8 && rb > (1 << 16)) return ORC_ERR_INVALID_ARG;
#pragma omp parallel for schedule(static) reduction(max : status)
    for (int t = 0; t < T; t++) {
        uint8_t qrow[1 << 16];   /* this token's fp8 row */
        const uint16_t* xrow = x + (int64_t)t * H;
        if (fmt == ORC_FMT_FP8) oracle_quantize_row(H, xrow, qrow);   /* once per token */
        for (int r = 0; r < R; r++) {
            int32_t s = send_slot[(int64_t)t * R + r];
            if (s < 0) continue;
            if (s >= capacity_rows) { status = ORC_ERR_CAPACITY; continue; }
            uint8_t* dst = send_buf + (int64_t)s * rb;
            if (fmt == ORC_FMT_BF16) memcpy(dst, xrow, (size_t)rb);
            else memcpy(dst, qrow, (size_t)rb);
            slot_src[s] = t;
            for (int j = 0; j < k; j++) {
                int e = topk_idx[(int64_t)t * k + j];
                int local = (e >= 0 && e / epr == r);
                slot_local_idx[(int64_t)s * k + j] = local ? e - r * epr : -1;
                slot_local_w[(int64_t)s * k + j] = local ? topk_w[(int64_t)t * k + j] : 0.0f;
            }
        }
    }
    return status;
}

/* ------------------------------------------------------------ descriptors
 * Closed form of the command stream ([UCCL] s2.3 WRITE fields, s3.1 message
 * types, s4.1 token packing, s4.2/s5.2 channels, s5.3 batch of 8):
 *   Reading: each rank's segment [o_r, o_{r+1}) is cut greedily into messages of
 *        at most 8 consecutive rows, starting at o_r;  message m of rank r is
 *        WRITE{dst_rank=r, src_offset=(o_r+8m)*row_bytes,
 *              dst_offset=8m*row_bytes, size=n*row_bytes, num_tokens=n}.
 *   Reading: after its WRITEs, each rank gets ATOMIC{dst_rank=r, op=ADD,
 *        value=cnt_r} (also when cnt_r = 0), so the receiver learns its count.
 *   Reading: dst_offset is relative to the start of rank r's receive region.
 *   Reading: rank r uses channel r mod C.
 * Records are emitted per channel c = 0..C-1, ranks ascending within the
 * channel, messages ascending, then the rank's ATOMIC.  Returns the number of
 * records (or -1 if max is too small). */
int64_t oracle_descriptors(int R, int C, const int32_t* num_tokens_per_rank,
                           const int32_t* rank_offset, int64_t row_bytes,
                           orc_cmd_t* out, int64_t max) {
    int64_t n = 0;
    for (int c = 0; c < C; c++) {
        for (int r = c; r < R; r += C) {
            int32_t cnt = num_tokens_per_rank[r];
            for (int32_t m = 0; 8 * m < cnt; m++) {
                int32_t rows = cnt - 8 * m;
                if (rows > 8) rows = 8;
                if (n >= max) return -1;
                orc_cmd_t d;
                memset(&d, 0, sizeof d);
                d.type = ORC_CMD_WRITE;
                d.op = 0;
                d.num_tokens = (uint16_t)rows;
                d.dst_rank = (uint32_t)r;
                d.size_or_value = (uint32_t)(rows * row_bytes);
                d.src_offset = (uint64_t)(rank_offset[r] + 8LL * m) * (uint64_t)row_bytes;
                d.dst_offset = (uint64_t)(8LL * m) * (uint64_t)row_bytes;
                out[n++] = d;
            }
            if (n >= max) return -1;
            orc_cmd_t a;
            memset(&a, 0, sizeof a);
            a.type = ORC_CMD_ATOMIC;
            a.op = ORC_ATOMIC_ADD;
            a.num_tokens = 0;
            a.dst_rank = (uint32_t)r;
            a.size_or_value = (uint32_t)cnt;
            out[n++] = a;
        }
    }
    return n;
}

/* ------------------------------------------------------------ combine
 * The returned expert outputs Y sit in the dispatch layout: row
 * send_slot[t,r] holds what rank r sends back for token t.  The combined
 * output is the gate-weighted sum over the token's destination ranks (reading):
 *   W[t,r]  = sum of w[t,j] over j with e_j != -1 and rank(e_j) = r
 *   out[t,h] = sum over r with send_slot[t,r] >= 0 of W[t,r] * Y[slot, h]
 * evaluated in double precision (the exact definition up to double rounding;
 * the GPU accumulates in float and stores bf16). */
void oracle_combine(int T, int H, int E, int R, int k, const uint16_t* y,
                    const int32_t* topk_idx, const float* topk_w,
                    const int32_t* send_slot, double* out) {
    int epr = E / R;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        double W[64];
        for (int r = 0; r < R; r++) W[r] = 0.0;
        for (int j = 0; j < k; j++) {
            int e = topk_idx[(int64_t)t * k + j];
            if (e < 0) continue;
            W[e / epr] += (double)topk_w[(int64_t)t * k + j];
        }
        double* o = out + (int64_t)t * H;
        for (int h = 0; h < H; h++) o[h] = 0.0;
        for (int r = 0; r < R; r++) {
            int32_t s = send_slot[(int64_t)t * R + r];
            if (s < 0) continue;
            const uint16_t* yrow = y + (int64_t)s * H;
            for (int h = 0; h < H; h++) o[h] += W[r] * (double)bf16_to_float(yrow[h]);
        }
    }
}

/* ------------------------------------------------------------ per-expert mode
 * The low-latency mode of [UCCL] s4.1 exchanges tokens per expert rather than
 * per rank: every kept choice (t, j) goes to the owner of expert e_j, into
 * that expert's receive rows ([GIN] s3.1.1: a token is sent to the owner of
 * its expert).  The pages give no layout; the readings are:
 *   Reading: no deduplication by rank; every (t, j) with e_j != -1 is one row,
 *        so a token that names an expert twice sends two rows.
 *   Reading: expert e's rows are [expert_offset[e], expert_offset[e+1]) of the
 *        send buffer, in ascending (t, j) order; expert_offset is the exclusive
 *        scan of num_tokens_per_expert (the same arrays as oracle_layout's).
 *   Reading: expert_slot[t, j] is the row of choice (t, j), or -1 if dropped. */
int oracle_ll_layout(int T, int E, int k, const int32_t* topk_idx,
                     int32_t* num_tokens_per_expert, int32_t* expert_offset,
                     int32_t* expert_slot) {
    if (T < 0 || E < 1 || E > 4096 || k < 1) return ORC_ERR_INVALID_ARG;
    int status = ORC_OK;
    for (int e = 0; e < E; e++) num_tokens_per_expert[e] = 0;
    for (int64_t i = 0; i < (int64_t)T * k; i++) {
        int e = topk_idx[i];
        if (e == -1) continue;
        if (e < -1 || e >= E) { status = ORC_ERR_BAD_EXPERT; continue; }
        num_tokens_per_expert[e]++;
    }
    int32_t acc = 0;   /* exclusive scan */
    for (int e = 0; e < E; e++) {
        expert_offset[e] = acc;
        acc += num_tokens_per_expert[e];
    }
    expert_offset[E] = acc;
    /* second pass: a running count per expert hands out the rows in order */
    int32_t run[4096];
    for (int e = 0; e < E; e++) run[e] = 0;
    for (int64_t i = 0; i < (int64_t)T * k; i++) {
        int e = topk_idx[i];
        if (e < 0 || e >= E) { expert_slot[i] = -1; continue; }
        expert_slot[i] = expert_offset[e] + run[e]++;
    }
    return status;
}

/* Row t (bf16, or its fp8 row) goes to send_buf row expert_slot[t, j] for
 * every kept choice.  Per-row metadata (reading): slot_src[s] = t and
 * slot_w[s] = w[t, j], the gate of that choice.  Rows at or beyond the
 * capacity are not written and ORC_ERR_CAPACITY is returned. */
int oracle_ll_pack(int T, int H, int k, int fmt, const uint16_t* x, const float* topk_w,
                   const int32_t* expert_slot, uint8_t* send_buf, int64_t capacity_rows,
                   int32_t* slot_src, float* slot_w) {
    if (fmt == ORC_FMT_FP8 && H % 128 != 0) return ORC_ERR_INVALID_ARG;
    int64_t rb = oracle_row_bytes(H, fmt);
    int status = ORC_OK;
    if (fmt == ORC_FMT_FP8 && rb > (1 << 16)) return ORC_ERR_INVALID_ARG;
#pragma omp parallel for schedule(static) reduction(max : status)
    for (int t = 0; t < T; t++) {
        uint8_t qbuf[1 << 16];   /* this token's fp8 row */
        const uint16_t* xrow = x + (int64_t)t * H;
        if (fmt == ORC_FMT_FP8) oracle_quantize_row(H, xrow, qbuf);
        for (int j = 0; j < k; j++) {
            int32_t s = expert_slot[(int64_t)t * k + j];
            if (s < 0) continue;
            if (s >= capacity_rows) { status = ORC_ERR_CAPACITY; continue; }
            uint8_t* dst = send_buf + (int64_t)s * rb;
            if (fmt == ORC_FMT_BF16) memcpy(dst, xrow, (size_t)rb);
            else memcpy(dst, qbuf, (size_t)rb);
            slot_src[s] = t;
            slot_w[s] = topk_w[(int64_t)t * k + j];
        }
    }
    return status;
}

/* Closed form of the per-expert command stream:
 *   Reading: each expert's rows are cut greedily into messages of at most 8
 *        consecutive rows ([UCCL] s4.1, s5.3); message m of expert e (on rank
 *        r = e / epr) is WRITE{dst_rank=r, src_offset=(eo_e+8m)*row_bytes,
 *        dst_offset=(eo_e - eo_{r*epr} + 8m)*row_bytes, size=n*row_bytes,
 *        num_tokens=n}: the destination keeps its experts' rows back to back.
 *   Reading: after its WRITEs, each expert (also one with no rows) gets
 *        ATOMIC{dst_rank=r, op=ADD, value=cnt_e, dst_offset=4*(e - r*epr)},
 *        which adds its count into the receiver's per-expert count word.
 *   Reading: rank r uses channel r mod C; per channel, ranks ascending, then
 *        the rank's experts ascending.
 * Returns the number of records, or -1 if max is too small. */
int64_t oracle_ll_descriptors(int E, int R, int C, const int32_t* num_tokens_per_expert,
                              const int32_t* expert_offset, int64_t row_bytes,
                              orc_cmd_t* out, int64_t max) {
    if (E % R != 0) return -1;
    int epr = E / R;
    int64_t n = 0;
    for (int c = 0; c < C; c++) {
        for (int r = c; r < R; r += C) {
            int32_t base = expert_offset[r * epr];
            for (int le = 0; le < epr; le++) {
                int e = r * epr + le;
                int32_t cnt = num_tokens_per_expert[e];
                for (int32_t m = 0; 8 * m < cnt; m++) {
                    int32_t rows = cnt - 8 * m < 8 ? cnt - 8 * m : 8;
                    if (n >= max) return -1;
                    orc_cmd_t d;
                    memset(&d, 0, sizeof d);
                    d.type = ORC_CMD_WRITE;
                    d.num_tokens = (uint16_t)rows;
                    d.dst_rank = (uint32_t)r;
                    d.size_or_value = (uint32_t)(rows * row_bytes);
                    d.src_offset = (uint64_t)(expert_offset[e] + 8LL * m) * (uint64_t)row_bytes;
                    d.dst_offset = (uint64_t)(expert_offset[e] - base + 8LL * m) * (uint64_t)row_bytes;
                    out[n++] = d;
                }
                if (n >= max) return -1;
                orc_cmd_t a;
                memset(&a, 0, sizeof a);
                a.type = ORC_CMD_ATOMIC;
                a.op = ORC_ATOMIC_ADD;
                a.dst_rank = (uint32_t)r;
                a.size_or_value = (uint32_t)num_tokens_per_expert[e];
                a.dst_offset = (uint64_t)(4 * le);
                out[n++] = a;
            }
        }
    }
    return n;
}

/* Per-expert combine: the expert outputs Y sit in the per-expert layout, row
 * expert_slot[t, j] holding expert e_j's output for token t.  The combined
 * output is the gate-weighted sum over the token's kept choices (the MoE
 * output by definition):
 *   out[t,h] = sum over j with e_j != -1 of w[t,j] * Y[expert_slot[t,j], h]
 * evaluated in double precision. */
void oracle_ll_combine(int T, int H, int k, const uint16_t* y, const int32_t* topk_idx,
                       const float* topk_w, const int32_t* expert_slot, double* out) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        double* o = out + (int64_t)t * H;
        for (int h = 0; h < H; h++) o[h] = 0.0;
        for (int j = 0; j < k; j++) {
            if (topk_idx[(int64_t)t * k + j] < 0) continue;
            int32_t s = expert_slot[(int64_t)t * k + j];
            if (s < 0) continue;
            double w = (double)topk_w[(int64_t)t * k + j];
            const uint16_t* yrow = y + (int64_t)s * H;
            for (int h = 0; h < H; h++) o[h] += w * (double)bf16_to_float(yrow[h]);
        }
    }
}
