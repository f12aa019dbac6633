/*
 * ep.h — C ABI of the MI355X (gfx950) MoE expert-parallel dispatch/combine
 * library: one GPU's share of an EP group, with the destination EP ranks
 * simulated as regions of the GPU's own HBM.
 *
 * Sources (page, section):
 *   UCCL-EP article (peacm.com/news/835744):
 *     s2.1  the GPU only writes a TransferCmd into a local FIFO and goes on
 *           computing; CPU proxy threads do the transfers;
 *     s2.2  FIFO ring {head, tail, slots, inflight_count}, lock-free head/tail
 *           with atomics, batched enqueue of up to 8 commands, non-blocking
 *           completion query, producer blocked at 256 commands in flight;
 *     s2.3  proxy loop: dequeue, switch on the type, WRITE ->
 *           PostRDMAWrite(dst_rank, src_offset, dst_offset, size);
 *     s3.1  the message types (Write, Atomic, Drain, Barrier);
 *     s3.2  an atomic carries an op and a value (4-bit op, 28-bit value);
 *     s4.1  low-latency mode: small tokens packed into one message; the
 *           dispatch kernel prepares the token data, synchronises, posts the
 *           transfer and goes on;
 *     s4.2  high-throughput mode: 8 independent FIFOs per GPU;
 *     s5.1  AMD port: 64-lane wavefronts instead of 32-lane warps;
 *     s5.2  tuning: FIFO depth 1024, 256 in flight, 8 channels, drain batch 32;
 *     s5.3  pack small messages with batch size 8;
 *     s6    EP32 dispatch and combine latencies.
 *   NCCL GIN article (bjdmk.com.cn/news/2086017):
 *     s2.2.1 caller-registered windows addressed by byte offsets;
 *     s3.1.1 device-side routing: each token goes to the owner of its expert;
 *     s4.2.1 error codes such as "window full".
 *   GPU communication notes (blog.zhenwei.site), s5: reuse long-lived
 *     buffers, keep explicit synchronisation boundaries; DeepEP dispatch and
 *     combine for MoE.
 *
 * Conventions for every call below:
 *   - Device pointers are HIP device allocations on the current device; the
 *     caller owns them and the stream.  The library never allocates device
 *     memory on the dispatch/combine path: scratch state comes in through
 *     `workspace` (size from ep_workspace_bytes) and the ring owns its own
 *     memory from ep_ring_create until ep_ring_destroy.
 *   - Calls enqueue kernels on `stream` and return at once with the result of
 *     host-side validation (EP_OK or EP_ERR_INVALID_ARG / EP_ERR_HIP).  Errors
 *     found on the device (bad expert id, capacity, ring timeout) are written to
 *     the device word `*dev_status` (int32, first error wins; the caller zeroes
 *     it and reads it after synchronising the stream).
 *   - Shapes: T tokens, H hidden size, E experts, R ranks, k experts per token.
 *     Requirements: T >= 0; H >= 8 and H % 8 == 0 (bf16) or H % 128 == 0
 *     (fp8); 1 <= R <= 64; E % R == 0; E <= 4096; 1 <= k <= min(E, 32);
 *     T * R < 2^31; T * max(k, R) < 2^31.
 *   - Expert e lives on rank e / (E / R).  A token goes once to every rank
 *     that owns one of its experts (the (token, rank) pair is the unit of
 *     dispatch).  Expert id -1 is a dropped choice and is skipped.
 *   - Alignment: x, send_buf, y, out and send_slot are 16-byte aligned,
 *     is_token_in_rank 4-byte aligned.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return value of every call and value of the device status word. */
enum ep_status {
    EP_OK = 0,
    EP_ERR_INVALID_ARG = 1,   /* host-side validation failed; nothing enqueued */
    EP_ERR_BAD_EXPERT = 2,    /* device: an expert id outside [-1, E) */
    EP_ERR_CAPACITY = 3,      /* device: P > capacity_rows */
    EP_ERR_RING_TIMEOUT = 4,  /* device: a producer waited longer than the ring's timeout */
    EP_ERR_HIP = 5,           /* a HIP runtime call failed */
    EP_ERR_BUSY = 6,          /* ring call not allowed while its proxy threads run */
    EP_ERR_TIMEOUT = 7        /* device: workgroups waited for each other too long */
};

/* Row format of the send buffer. */
enum ep_format {
    EP_FMT_BF16 = 0,           /* a row is the token's H bf16 values: 2H bytes */
    EP_FMT_FP8_E4M3_B128 = 1   /* H OCP e4m3 codes, H/128 float scales, zero pad
                                  to a multiple of 128 bytes */
};

/* TransferCmd types (UCCL-EP s3.1) and atomic ops (s3.2). */
enum { EP_CMD_WRITE = 1, EP_CMD_ATOMIC = 2 };
enum { EP_ATOMIC_ADD = 1 };

typedef struct ep_shape {
    int32_t T, H, E, R, k, fmt;
} ep_shape_t;

/* One TransferCmd, 32 bytes: the command a CPU proxy would execute
 * (UCCL-EP s2.3 WRITE fields; s3.2 op/value), as returned by the drain and
 * proxy calls.  `seq` is the command's ticket in its channel + 1 (its FIFO
 * position).  In the ring itself the GPU stores each command as four
 * self-tagged 8-byte words, so it never writes a separate ready flag.
 *   WRITE : copy `size_or_value` bytes holding `num_tokens` (1..8) rows from
 *           byte `src_offset` of the send buffer to byte `dst_offset` of rank
 *           `dst_rank`'s receive region.
 *   ATOMIC: add `size_or_value` (the rank's row count, < 2^28) to rank
 *           `dst_rank`'s count word; follows all of that rank's WRITEs in
 *           its channel. */
typedef struct ep_transfer_cmd {
    uint32_t seq;
    uint8_t type;
    uint8_t op;
    uint16_t num_tokens;
    uint32_t dst_rank;
    uint32_t size_or_value;
    uint64_t src_offset;
    uint64_t dst_offset;
} ep_transfer_cmd_t;

typedef struct ep_ring ep_ring_t;

/* Bytes of one send-buffer row (the row pitch): 2H for bf16; for fp8,
 * H + 4*(H/128) rounded up to a multiple of 128 (7424 at H = 7168), the bytes
 * after the scales being zero. */
size_t ep_row_bytes(int32_t H, int32_t fmt);

/* Bytes of device workspace that ep_dispatch_layout and ep_dispatch need for
 * `shape` (grid-barrier words, per-tile partial counts, per-message
 * arrival counters).  One workspace serves a layout call and the dispatch
 * calls that follow it on the same stream.  It must be zero-filled once
 * before its first use (e.g. hipMemset); the library leaves it consistent
 * after every call that completes.  A workspace sized for a shape also serves
 * every smaller shape.  After a call fails with EP_ERR_TIMEOUT it must be
 * zero-filled again.  Returns 0 for an invalid shape. */
size_t ep_workspace_bytes(const ep_shape_t* shape);

/* Routing layout.  UCCL-EP s1 (token-level exchange with many
 * peers), NCCL GIN s3.1.1 (each token is routed to the owner of its expert).
 *   topk_idx              int32 [T,k]   expert ids, -1 = dropped
 *   num_tokens_per_rank   int32 [R]     cnt_r = #tokens with >= 1 expert on r
 *   num_tokens_per_expert int32 [E]     cnt_e = #(t,j) with topk_idx = e
 *   rank_offset           int32 [R+1]   exclusive scan of cnt_r; P = rank_offset[R]
 *   expert_offset         int32 [E+1]   exclusive scan of cnt_e
 *   is_token_in_rank      uint8 [T,R]   1 if token t goes to rank r
 *   send_slot             int32 [T,R]   row of (t,r) in the send buffer, or -1;
 *                                       rank r's rows are [o_r, o_{r+1}) in
 *                                       ascending token order
 * Device errors: EP_ERR_BAD_EXPERT (the offending entry is skipped),
 * EP_ERR_TIMEOUT (the tiles of the one-kernel layout did not all become
 * resident within a second; outputs are then unspecified). */
int ep_dispatch_layout(const ep_shape_t* shape, const int32_t* topk_idx,
                       int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                       int32_t* rank_offset, int32_t* expert_offset,
                       uint8_t* is_token_in_rank, int32_t* send_slot,
                       void* workspace, size_t workspace_bytes,
                       int32_t* dev_status, hipStream_t stream);

/* Pack and descriptor emission.  UCCL-EP s4.1 (prepare the
 * token data, then post the transfer), s2.2 (FIFO), s4.2/s5.2 (channels).
 * Must follow ep_dispatch_layout on the same stream with the same workspace.
 *   x              bf16 [T,H]           token rows
 *   topk_idx/_w    int32/float [T,k]    routing and gate weights
 *   rank_offset, send_slot              from ep_dispatch_layout
 *   send_buf       [capacity_rows, ep_row_bytes(H, fmt)]  rank-contiguous rows;
 *                  for fp8 each row is quantised once per token: per 128-element
 *                  block a = max(max|x|, 1e-4), codes e4m3(x * (448/a)) with
 *                  round-to-nearest-even and saturation, scale a/448.  A NaN
 *                  element takes no part in max|x|; an infinite one makes a
 *                  and the scale infinite; a NaN product gets code 0x7F with
 *                  the element's sign
 *   slot_src       int32 [capacity_rows]    token of each row
 *   slot_local_idx int32 [capacity_rows,k]  e_j - r*E/R if e_j is on the row's
 *                                           rank r, else -1
 *   slot_local_w   float [capacity_rows,k]  w_j if e_j is on r, else 0
 *   ring           may be NULL (no descriptors).  Otherwise, per rank r, rows
 *                  [o_r, o_{r+1}) are cut into messages of <= 8 rows, each a
 *                  WRITE published on channel r % channels only after its rows
 *                  are written (system-scope release), followed by one
 *                  ATOMIC ADD of cnt_r (also for cnt_r = 0).
 * Device errors: EP_ERR_CAPACITY (rows >= capacity_rows are not written and
 * no descriptor is emitted), EP_ERR_RING_TIMEOUT (the ring stayed full for
 * longer than its timeout), EP_ERR_INVALID_ARG (send_slot and rank_offset do
 * not come from the same layout; a group of rows found inconsistent publishes
 * nothing).  A status already set when the call starts (e.g. a bad expert id
 * from the layout) means no descriptor is emitted.  After any device error
 * on a call with a ring, the ring may hold tickets that were reserved but
 * never written, where a consumer would wait: stop the proxy threads and call
 * ep_ring_reset before the ring is used again. */
int ep_dispatch(const ep_shape_t* shape, const void* x, const int32_t* topk_idx,
                const float* topk_w, const int32_t* rank_offset, const int32_t* send_slot,
                void* send_buf, int64_t capacity_rows,
                int32_t* slot_src, int32_t* slot_local_idx, float* slot_local_w,
                ep_ring_t* ring, void* workspace, size_t workspace_bytes,
                int32_t* dev_status, hipStream_t stream);

/* Layout and pack in one call: the outputs of ep_dispatch_layout followed by
 * ep_dispatch, with the same arguments, meanings and device errors (and
 * EP_ERR_TIMEOUT as for ep_dispatch_layout).  UCCL-EP s4.1 (the dispatch
 * prepares the token data, synchronises, then posts the transfers; for small
 * decode batches latency, not bandwidth, is the cost).  For T <= 256 it is
 * one kernel: every workgroup derives the whole (small) layout from topk_idx
 * on chip and starts copying rows at once, and the descriptors are published
 * in closed form by the last workgroup to finish its rows.  For T >= 1024
 * with bf16 rows that one wavefront covers (H in (1024, 8192]) it is one
 * kernel too, when its workgroups can all be resident and the batch is not
 * so long that ep_dispatch would give each row two wavefronts (whole rows
 * making 4 or more passes over the chip): each workgroup computes the rank
 * ballots of its own tokens' 64-token blocks, they meet at a grid barrier,
 * and each derives its slots from a per-block count table, then packs and
 * publishes as ep_dispatch does.  Otherwise it makes the two calls.
 * ep_dispatch_fused_plan says which.
 * send_slot must be 16-byte and is_token_in_rank 4-byte aligned when
 * T > 256.  Leaves in the workspace what a following ep_dispatch with the
 * same layout needs, but not the per-tile expert counts that
 * ep_dispatch_layout_ll reads (that one follows ep_dispatch_layout). */
int ep_dispatch_fused(const ep_shape_t* shape, const void* x, const int32_t* topk_idx,
                      const float* topk_w, int32_t* num_tokens_per_rank,
                      int32_t* num_tokens_per_expert, int32_t* rank_offset,
                      int32_t* expert_offset, uint8_t* is_token_in_rank, int32_t* send_slot,
                      void* send_buf, int64_t capacity_rows,
                      int32_t* slot_src, int32_t* slot_local_idx, float* slot_local_w,
                      ep_ring_t* ring, void* workspace, size_t workspace_bytes,
                      int32_t* dev_status, hipStream_t stream);

/* Which path ep_dispatch_fused takes for `shape` on the current device, for
 * a call with a ring (with_ring != 0) or without: EP_FUSED_ONE_KERNEL_SMALL,
 * EP_FUSED_ONE_KERNEL_LARGE or EP_FUSED_TWO_CALLS; EP_ERR_INVALID_ARG for an
 * invalid shape.  Launches nothing. */
enum {   /* distinct from every status code */
    EP_FUSED_ONE_KERNEL_SMALL = 101,
    EP_FUSED_ONE_KERNEL_LARGE = 102,
    EP_FUSED_TWO_CALLS = 103
};
int ep_dispatch_fused_plan(const ep_shape_t* shape, int32_t with_ring);

/* ep_dispatch_fused for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments (minus the workspace), outputs,
 * meanings and device errors as ep_dispatch_fused.  Its scratch is a 4 MiB
 * device array inside the library, one per GPU, held until the process ends;
 * the call allocates nothing.  Shapes whose ep_workspace_bytes exceed 4 MiB
 * are rejected with EP_ERR_INVALID_ARG before anything is enqueued
 * (ep_last_error says why).  The first call on each GPU zero-fills that
 * GPU's array with a kernel on `stream`; clear_scratch != 0 does it again
 * (needed only after a call reported EP_ERR_TIMEOUT).  Every call on a GPU
 * shares its array: calls on one GPU must be ordered (one stream, or
 * synchronised); calls that overlap in time race. */
int ep_dispatch_fused_noalloc(const ep_shape_t* shape, const void* x, const int32_t* topk_idx,
                              const float* topk_w, int32_t* num_tokens_per_rank,
                              int32_t* num_tokens_per_expert, int32_t* rank_offset,
                              int32_t* expert_offset, uint8_t* is_token_in_rank,
                              int32_t* send_slot, void* send_buf, int64_t capacity_rows,
                              int32_t* slot_src, int32_t* slot_local_idx, float* slot_local_w,
                              ep_ring_t* ring, int32_t clear_scratch, int32_t* dev_status,
                              hipStream_t stream);

/* Combine.  UCCL-EP s6 (EP combine), GPU communication notes s5
 * (DeepEP combine).  The returned expert outputs y sit in the dispatch
 * layout: y row send_slot[t,r] is rank r's result for token t.
 *   W[t,r]   = sum of w[t,j] (float adds, ascending j) over j with
 *              e_j != -1 on rank r
 *   out[t,:] = bf16_rne( sum over ranks r ascending with send_slot[t,r] >= 0
 *              of W[t,r] * y[send_slot[t,r], :] ), accumulated with float fma
 *   y   bf16 [y_rows,H] (y_rows >= P), out bf16 [T,H].  Tokens with no
 *       destination get zeros.
 * Device error: EP_ERR_CAPACITY if a slot is >= y_rows (that row is skipped). */
int ep_combine(const ep_shape_t* shape, const void* y, int64_t y_rows,
               const int32_t* topk_idx, const float* topk_w, const int32_t* send_slot,
               void* out, int32_t* dev_status, hipStream_t stream);

/* ---- Per-expert (low-latency) mode ------------------------------------------
 * UCCL-EP s4.1 (low-latency mode: tokens are exchanged per expert, for small
 * batches), NCCL GIN s3.1.1 (a token is sent to the owner of its expert).
 * Every kept choice (t, j) (e_j != -1) is one row; no deduplication by rank,
 * so a token naming an expert twice sends two rows.  Q = expert_offset[E] =
 * the number of kept choices.  Expert e's rows are [expert_offset[e],
 * expert_offset[e+1]) in ascending (t, j) order; since the experts of a rank
 * are contiguous, so are a rank's rows. */

/* The row of every choice: expert_slot[t*k + j] = expert_offset[e] + the
 * number of kept choices (t', j') < (t, j) in (t, j) order naming the same
 * expert e = topk_idx[t,j]; -1 for a dropped choice (or a bad id, reported as
 * EP_ERR_BAD_EXPERT).
 *   expert_offset int32 [E+1]  from ep_dispatch_layout
 *   expert_slot   int32 [T,k]  output
 * Must follow ep_dispatch_layout on the same stream with the same topk_idx
 * and workspace: it reads the per-tile expert count prefixes left there. */
int ep_dispatch_layout_ll(const ep_shape_t* shape, const int32_t* topk_idx,
                          const int32_t* expert_offset, int32_t* expert_slot,
                          void* workspace, size_t workspace_bytes,
                          int32_t* dev_status, hipStream_t stream);

/* The whole per-expert layout in one call, without the rank layout: the
 * outputs num_tokens_per_expert [E] and expert_offset [E+1] of
 * ep_dispatch_layout and expert_slot [T,k] of ep_dispatch_layout_ll, with the
 * same meanings and device errors (EP_ERR_BAD_EXPERT: the entry is treated as
 * dropped; EP_ERR_TIMEOUT: the tiles did not all become resident within a
 * second).  One kernel: tiles of 256 tokens count their choices per expert,
 * meet at a grid barrier, and each derives its rows from the tiles' counts.
 * UCCL-EP s4.1 (low-latency mode: tokens go per expert).  Only for
 * E <= 1024 and as many tiles as the device holds at once (ceil(T/256) up to a
 * few hundred on MI355X); otherwise EP_ERR_INVALID_ARG with nothing enqueued
 * (ep_last_error says why) and ep_dispatch_layout + ep_dispatch_layout_ll
 * serve.  Leaves the workspace ready for ep_dispatch_ll. */
int ep_dispatch_ll_layout(const ep_shape_t* shape, const int32_t* topk_idx,
                          int32_t* num_tokens_per_expert, int32_t* expert_offset,
                          int32_t* expert_slot, void* workspace, size_t workspace_bytes,
                          int32_t* dev_status, hipStream_t stream);

/* Per-expert pack and descriptors.  Row expert_slot[t,j] of send_buf gets
 * x[t] (bf16, or its fp8 row as in ep_dispatch); metadata slot_src[s] = t and
 * slot_w[s] = w[t,j] (the gate of that choice).  Must follow the per-expert
 * layout (ep_dispatch_layout + ep_dispatch_layout_ll, or
 * ep_dispatch_ll_layout) on the same stream with the same workspace.
 *   send_buf [capacity_rows, row bytes], 16-byte aligned; capacity_rows >= Q
 *   slot_src int32 [capacity_rows], slot_w float [capacity_rows]
 *   ring     may be NULL.  Otherwise, per expert e on rank r = e / (E/R), its
 *            rows are cut into messages of <= 8 rows: WRITE{dst_rank r,
 *            src_offset (expert_offset[e] + 8m) * row bytes, dst_offset
 *            (expert_offset[e] - expert_offset[r*E/R] + 8m) * row bytes}, then
 *            ATOMIC{ADD, value cnt_e, dst_offset 4 * (e - r*E/R)} (the
 *            receiver's count word of that expert; also for cnt_e = 0).  Rank
 *            r uses channel r % channels.  A WRITE is published only after
 *            its rows are written (visible to other agents), an expert's
 *            ATOMIC after all of its WRITEs.  Small batches (fewer than 1024
 *            row chunks) publish in closed form once every row is written:
 *            per channel, ranks ascending, a rank's experts ascending; larger
 *            ones as each message's rows complete.
 * Device errors: EP_ERR_CAPACITY (rows >= capacity_rows are not written, no
 * descriptor is emitted), EP_ERR_RING_TIMEOUT, EP_ERR_INVALID_ARG
 * (expert_slot and expert_offset do not come from the same layout; no
 * descriptor is emitted). */
int ep_dispatch_ll(const ep_shape_t* shape, const void* x, const int32_t* topk_idx,
                   const float* topk_w, const int32_t* expert_offset,
                   const int32_t* expert_slot, void* send_buf, int64_t capacity_rows,
                   int32_t* slot_src, float* slot_w, ep_ring_t* ring, void* workspace,
                   size_t workspace_bytes, int32_t* dev_status, hipStream_t stream);

/* Per-expert layout, row table and pack in one call, for small decode
 * batches: the outputs num_tokens_per_expert, expert_offset and expert_slot
 * of ep_dispatch_layout + ep_dispatch_layout_ll, and the rows, metadata and
 * descriptors of ep_dispatch_ll, with the same meanings and device errors.
 * UCCL-EP s4.1 (the low-latency mode serves small batches, where latency is
 * the cost).  One kernel: every workgroup derives the row table on chip and
 * starts copying at once; the last workgroup to finish its rows publishes in
 * closed form.  The rank-layout outputs are not produced.  Only for
 * T <= 256 and E <= 1024 (else EP_ERR_INVALID_ARG, nothing launched). */
int ep_dispatch_ll_fused(const ep_shape_t* shape, const void* x, const int32_t* topk_idx,
                         const float* topk_w, int32_t* num_tokens_per_expert,
                         int32_t* expert_offset, int32_t* expert_slot,
                         void* send_buf, int64_t capacity_rows, int32_t* slot_src, float* slot_w,
                         ep_ring_t* ring, void* workspace, size_t workspace_bytes,
                         int32_t* dev_status, hipStream_t stream);

/* Per-expert combine: y row expert_slot[t,j] is expert e_j's output for
 * token t, and
 *   out[t,:] = bf16_rne( sum over kept j ascending of w[t,j] * y[expert_slot[t,j], :] )
 * accumulated with float fma.  y bf16 [y_rows,H] (y_rows >= Q), out bf16
 * [T,H].  Device error: EP_ERR_CAPACITY if a row is >= y_rows (skipped). */
int ep_combine_ll(const ep_shape_t* shape, const void* y, int64_t y_rows,
                  const int32_t* topk_idx, const float* topk_w, const int32_t* expert_slot,
                  void* out, int32_t* dev_status, hipStream_t stream);

/* ---- TransferCmd ring (UCCL-EP s2.2, s2.3, s5.2) ---------------------------
 * `channels` FIFOs of `depth` slots each; a producer blocks while
 * `max_inflight` commands of its channel are published but not yet drained,
 * and gives up with EP_ERR_RING_TIMEOUT after `timeout_ns`.  Slots and the
 * consumer position live in host-pinned coherent memory (the consumer is a
 * CPU proxy); the producer ticket counter and a cached copy of the consumer
 * position live in device memory.  Allocated on the current device; returns
 * NULL on invalid arguments (depth < 1 or > 65535, channels < 1 or > 64,
 * max_inflight < 1 or > depth, timeout_ns < 1) or allocation failure.
 * Descriptor offsets must fit 48 bits (capacity_rows * row bytes < 2^48).
 * A ring serves one stream at a time. */
ep_ring_t* ep_ring_create(int32_t depth, int32_t channels, int32_t max_inflight,
                          int64_t timeout_ns);
int ep_ring_destroy(ep_ring_t* ring);

/* Host-only, while no kernel uses the ring and no proxy runs: clear slots,
 * tickets and positions.  Required after a dispatch on the ring reported a
 * device error. */
int ep_ring_reset(ep_ring_t* ring);

/* Stand-in for one proxy dequeue: pop up to `max` published commands of
 * `channel` in FIFO order into `out`, mark them completed and return their
 * number in *n_out.  EP_ERR_BUSY while proxy threads run. */
int ep_ring_drain(ep_ring_t* ring, int32_t channel, ep_transfer_cmd_t* out,
                  int32_t max, int32_t* n_out);

/* Proxy threads (UCCL-EP s2.3): `threads` host threads poll the channels
 * (thread i serves channels i, i+threads, ...), pop commands in batches of
 * up to 32, mark them completed and append them to a log of `log_capacity`
 * entries (further commands are counted, not logged). */
int ep_ring_proxy_start(ep_ring_t* ring, int32_t threads, int64_t log_capacity);

/* Stop the proxy threads after they have drained every command published so
 * far; copy up to `log_max` logged commands into `log_out` (may be NULL) and
 * return the number logged and drained in *n_logged and *n_drained. */
int ep_ring_proxy_stop(ep_ring_t* ring, ep_transfer_cmd_t* log_out, int64_t log_max,
                       int64_t* n_logged, int64_t* n_drained);

/* Commands drained so far by the proxy threads (a live counter). */
int64_t ep_ring_proxy_drained(const ep_ring_t* ring);

/* Loopback execution target (UCCL-EP s2.3: the proxy executes each command it
 * pops; s2.2: completions are tracked per command).  Host-only, while no
 * proxy runs.  With src set, proxy threads started afterwards execute what
 * they pop, each on its own stream, in ticket order per channel.  A popped
 * command's slot goes back to the producers at once (the in-flight limit
 * counts published, not yet popped commands), but its copy reads the send
 * buffer later: the caller must not rewrite the send buffer (e.g. by the
 * next dispatch into it) before ep_ring_wait_complete has returned.
 *   WRITE       copy size_or_value bytes from src + src_offset to
 *               dst[dst_rank] + dst_offset (device to device); consecutive
 *               WRITEs that continue each other become one copy;
 *   ATOMIC ADD  add value to the int32 at counts[dst_rank] + dst_offset.
 * A command is completed once its copy or add has finished.  Commands that
 * fall outside the registered byte ranges (src_bytes, dst_bytes[r],
 * count_bytes[r]) are skipped and counted as errors.  dst, dst_bytes, counts
 * and count_bytes are host arrays of R entries (device pointers may be NULL
 * with size 0); they are copied.  src = NULL switches loopback off. */
int ep_ring_set_loopback(ep_ring_t* ring, const void* src, uint64_t src_bytes, int32_t R,
                         void* const* dst, const uint64_t* dst_bytes, void* const* counts,
                         const uint64_t* count_bytes);

/* Commands of `channel` completed so far (-1 on bad arguments); a command
 * with ticket t (its seq - 1) is complete once this exceeds t. */
int64_t ep_ring_completed(const ep_ring_t* ring, int32_t channel);

/* CheckCompletion on the GPU (UCCL-EP s2.2: a command's completion can be
 * queried without blocking).  Enqueues on `stream` one kernel that, for
 * i < n, writes done[i] = 1 if the command with ticket tickets[i] (its seq -
 * 1) on channel channels[i] has completed, 0 if not yet, 2 if the channel is
 * not one of the ring's.  The proxy threads (or ep_ring_drain) keep each
 * channel's completed count in host-pinned memory that the kernel reads; a
 * channel's commands complete in ticket order.  The kernel never waits.
 *   channels int32 [n], tickets uint64 [n], done uint8 [n]: device memory.
 * Returns EP_ERR_INVALID_ARG for a NULL ring or n < 0. */
int ep_ring_check_completion(const ep_ring_t* ring, const int32_t* channels,
                             const uint64_t* tickets, int32_t n, uint8_t* done,
                             hipStream_t stream);

/* Block the calling host thread until every command published so far (the
 * producers' ticket counters, read from the device) is completed.  Call it
 * after the dispatch that published them has finished.  EP_ERR_RING_TIMEOUT
 * after timeout_ns; EP_ERR_INVALID_ARG if loopback execution skipped a
 * command (see ep_ring_set_loopback). */
int ep_ring_wait_complete(ep_ring_t* ring, int64_t timeout_ns);

/* Loopback counters since ep_ring_set_loopback: commands completed, commands
 * skipped as errors, copies issued (after merging), and the mean and largest
 * time from a command's pop to its completion, in microseconds. */
int ep_ring_loopback_stats(const ep_ring_t* ring, int64_t* n_done, int64_t* n_errors,
                           int64_t* n_copies, double* mean_latency_us, double* max_latency_us);

/* Text of a status code. */
const char* ep_status_str(int status);

/* Description of the last HIP runtime failure seen by this library on the
 * calling thread (the call that returned EP_ERR_HIP), or of the last host-side
 * rejection that records a reason, or "" if none. */
const char* ep_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
