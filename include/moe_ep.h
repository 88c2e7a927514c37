/*
 * moe_ep.h -- C ABI of libmoe_ep: MoE expert-parallel dispatch / combine on
 * one AMD Instinct MI355X (gfx950), with all N logical EP ranks in one HBM.
 *
 * Operations (source: "Enabling trillion-parameter models on AWS EFA",
 * Perplexity 2025):
 *   - dispatch splits each rank's tokens and sends every token to the ranks
 *     hosting its top-k experts; combine brings the processed rows back and
 *     forms each token's weighted average (section "Introduction");
 *   - both are split into a send half and a receive half (section "EFA-based
 *     MoE all-to-all");
 *   - senders count tokens per expert, exchange the counts, and an exclusive
 *     prefix sum gives every sender conflict-free, contiguous write offsets;
 *     a receive region holds at most N*T*max(k, E/N) rows (section "Send and
 *     receive buffers");
 *   - the receive half shuffles the receive buffer into the tensor a grouped
 *     GEMM consumes; combine accumulates the k rows of a token on the receive
 *     side (section "Dispatch and combine");
 *   - dispatch payload is block-scaled fp8, combine payload bf16 (section
 *     "Evaluation: dispatch/combine latency").
 * On one GPU a "remote write" into rank d is a store into rank d's region of
 * the same HBM; the N ranks are stacked on a leading axis and one call covers
 * all of them.
 *
 * Conventions shared by every call
 *   - All array arguments are DEVICE pointers owned by the caller; the library
 *     allocates nothing and keeps no state between calls except the caller's
 *     workspace.  bf16 arrays are passed as uint16_t (raw bfloat16 bits).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; nothing waits for the GPU except
 *     moe_status().  Calls that share a workspace must be ordered on one stream.
 *   - Return value: MOE_OK, or a negative MOE_E* code when the arguments are
 *     rejected on the host, in which case nothing was enqueued.
 *   - Errors found on the GPU (bad expert ids, region overflow) never cause an
 *     out-of-bounds access: the offending row is dropped and a sticky bit is
 *     set in the workspace's error word, read and cleared by moe_status().
 *
 * Layout readings (the pages leave these open):
 *   - expert e lives on rank e / L, L = E / N (contiguous blocks);
 *   - inside one (source rank, expert) group rows keep ascending
 *     (token, slot) order, so every position is unique;
 *   - receive region d holds one contiguous block per source rank, sources
 *     in ascending order, each block in the sender's (expert, token, slot)
 *     order;
 *   - the grouped-GEMM layout of rank d is expert-major, (source, token, slot)
 *     ascending inside an expert, no padding between experts;
 *   - a token sends one row per (token, slot).
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Host-side return codes. */
#define MOE_OK 0
#define MOE_EINVAL (-1) /* shape or argument outside the supported domain   */
#define MOE_ENULL (-2)  /* a required pointer is NULL                        */
#define MOE_EALIGN (-3) /* a pointer is not aligned as documented            */
#define MOE_ERANGE (-4) /* a row count or size does not fit the index types   */
#define MOE_EHIP (-5)   /* the HIP runtime refused a launch or a copy         */

/* Sticky device-side error bits (moe_status). */
#define MOE_FLAG_BADID 1u    /* a top-k id outside [0, E): that slot was dropped  */
#define MOE_FLAG_OVERFLOW 2u /* a fixed region got more rows than region_rows     */
#define MOE_FLAG_BOUND 4u    /* a region count exceeded N*T*max(k, E/N)           */
#define MOE_FLAG_TIMEOUT 8u  /* moe_dispatch_send_ll / moe_dispatch_direct_ll: a wait
                                inside the launch gave up (its rows were dropped);
                                re-initialise ws                                  */

/*
 * Problem shape, per logical rank, identical on all N ranks.
 *   N            logical EP ranks, 1..256
 *   T            tokens per rank, 0..2^31-1
 *   H            hidden size: multiple of 128, 128..32768
 *   E            experts: multiple of N, at most 1024
 *   k            experts per token: 1..min(E, 64)
 *   region_rows  0 = packed receive regions: region d starts right after
 *                region d-1 and the arrays hold exactly N*T*k rows;
 *                R > 0 = fixed regions: region d is rows [d*R, d*R + R)
 *                and the arrays hold N*R rows.  R = N*T*max(k, E/N) is the
 *                worst-case bound of "Send and receive buffers" and never
 *                overflows.
 *   early_rows   C > 0 (fixed regions only, N*C <= R): region d starts with
 *                C private rows per sender ("Send and receive buffers": a
 *                little private per-sender space on every receiver lets
 *                some tokens go out before the count exchange).  Sender s's
 *                first C rows for d go to region rows s*C .. s*C + C - 1 in
 *                its sender order, a place it knows without the exchange;
 *                its further rows follow from region row N*C, stacked by
 *                source.  The expert-major layout does not change.
 * N*T*k and N*R must stay below 2^31.
 */
typedef struct moe_shape {
  int32_t N, T, H, E, k;
  int32_t early_rows; /* C: private rows per sender in every fixed region, 0 = none */
  int64_t region_rows;
} moe_shape;

/* Rows every receive / expert-major array must hold (N*T*k packed, N*R fixed);
 * negative MOE_E* code for a rejected shape. */
int64_t moe_recv_rows(const moe_shape *shape);

/* Bytes of workspace the calls need for `shape` (negative MOE_E* if rejected).
 * The workspace holds per-chunk and per-rank counts, all offsets, the region
 * bases and the sticky error word. */
int64_t moe_workspace_bytes(const moe_shape *shape);

/* Zero the workspace header (the error word) and, when every rank fits one
 * routing chunk (T*k <= 4096), the exchange area of the single-launch calls.
 * Call once after allocating a workspace, before its first use, and again
 * before using it for another shape.  ws: device, 256-B aligned. */
int moe_workspace_init(const moe_shape *shape, void *ws, void *stream);

/*
 * Dispatch, send half ("Dispatch and combine"): per-expert counts with LDS
 * atomics, the count exchange and exclusive prefix sums, stable slot
 * positions, then quantisation and the stores into every destination's
 * receive region.
 *   tokens    bf16 [N][T][H], 16-B aligned.  May be NULL: then only the
 *             routing layout (workspace, send_pos) is produced and no payload
 *             is written (a combine-only setup).
 *   topk_idx  int32 [N][T][k]: expert of slot j of token t on rank s.
 *   recv_q    fp8 e4m3fn [rows][H] (rows = moe_recv_rows), 16-B aligned:
 *             receive regions, source-major.  Slot (s,t,j) with expert e on
 *             rank d = e/L and block index u = send_pos[s][t][j] -
 *             send_off[s][d*L] lands at row base[d] + recv_off[d][s] + u
 *             (with early rows C: base[d] + s*C + u if u < C, else
 *             base[d] + N*C + recv_off[d][s] + u - C).
 *   recv_s    fp32 [rows][H/128]: the scale of each 128-element block,
 *             scale = amax/448 (IEEE division), q = e4m3fn_rne_satfinite
 *             (x/scale); an all-zero block has scale 0 and zero bytes.
 *   send_pos  int32 [N][T][k] out: position of each slot in its sender's
 *             (expert, token, slot) order; -1 for a dropped (bad id) slot.
 *   ws        workspace of moe_workspace_bytes(shape), initialised once.
 * Rows of the arrays that no slot fills are left untouched.
 */
int moe_dispatch_send(const moe_shape *shape, const uint16_t *tokens, const int32_t *topk_idx,
                      uint8_t *recv_q, float *recv_s, int32_t *send_pos, void *ws, void *stream);

/*
 * Dispatch, send half, in ONE kernel launch (AWS China blog "750B MoE model
 * migration from a self-built RoCE cluster to AWS EFA", section 4.4, DeepEP
 * low-latency mode: the whole dispatch in a single kernel with no CPU
 * involvement, for small decode batches).  Same arguments and the same
 * results, bit for bit, as moe_dispatch_send, including every table that
 * moe_dispatch_recv, moe_combine_pull and moe_layout_export read from ws.
 * Counting, the count exchange, the scans and the quantised stores run in
 * one grid; workgroups hand values to each other through ws (each value
 * tagged with a per-workspace call number that the launch advances), so:
 *   - every rank's slots must fit one routing chunk: T*k <= 4096, else
 *     MOE_EINVAL (use moe_dispatch_send);
 *   - ws must have been initialised by moe_workspace_init for this shape;
 *     calls on one workspace must not overlap (one stream);
 *   - every wait inside the launch is bounded; a wait that gives up sets
 *     MOE_FLAG_TIMEOUT and drops the rows that depended on it (never seen in
 *     correct use; re-initialise ws afterwards).
 */
int moe_dispatch_send_ll(const moe_shape *shape, const uint16_t *tokens, const int32_t *topk_idx,
                         uint8_t *recv_q, float *recv_s, int32_t *send_pos, void *ws, void *stream);

/*
 * Dispatch in one call, straight into the grouped-GEMM layout ("Dispatch and
 * combine": peers whose buffers are mapped can push tokens directly; on one
 * GPU every rank is such a peer).  The same results as moe_dispatch_send
 * followed by moe_dispatch_recv -- send_pos, x_q, x_s, exp_off, row_src and
 * the workspace tables, bit for bit -- but each quantised row is stored
 * once, at its expert-major row, and no source-major receive region is
 * written or read.
 *   tokens    bf16 [N][T][H], 16-B aligned, or NULL (layout only: send_pos,
 *             exp_off, row_src).
 *   topk_idx  int32 [N][T][k].
 *   x_q, x_s  out, fp8 [rows][H] and fp32 [rows][H/128], as from
 *             moe_dispatch_recv (NULL with tokens NULL).
 *   send_pos, exp_off, row_src   out, as from moe_dispatch_send /
 *             moe_dispatch_recv.
 *   ws        workspace of moe_workspace_bytes(shape), initialised once.
 */
int moe_dispatch_direct(const moe_shape *shape, const uint16_t *tokens, const int32_t *topk_idx, uint8_t *x_q,
                        float *x_s, int32_t *send_pos, int32_t *exp_off, int32_t *row_src, void *ws, void *stream);

/*
 * moe_dispatch_direct without a caller workspace, for callers that cannot
 * allocate device memory (code under graph capture, serving loops or
 * harnesses that forbid hipMalloc): the routing tables live in a 32 MiB
 * device array of the library's own, one per GPU, set aside when the
 * library is loaded and held until the process ends.  Nothing is allocated
 * by the call.  Same arguments, results and limits as moe_dispatch_direct
 * (bit for bit), with ws replaced by
 *   flags   uint32 out, device, 4-B aligned: the sticky error bits of this
 *           call (MOE_FLAG_*), written when the call's work completes.
 * The tables take about 4 bytes per slot (N*T*k) once a rank has more than
 * 4096 slots, plus about 4*N*E*(B + 4) bytes with B = the rank's routing
 * chunks of up to 4096 slots; a shape whose tables exceed 32 MiB is rejected
 * with MOE_ERANGE before anything is enqueued (a prefill chunk of N = 8,
 * T = 16384, k = 8, E = 256 needs 4.3 MiB).  Every call on one GPU uses the
 * same array: calls that overlap on one GPU (on different streams) race and
 * must not be issued; calls on one stream are ordered.  Unlike
 * moe_dispatch_direct, no workspace tables remain for later calls
 * (moe_combine_pull, moe_layout_export): the outputs are complete on their
 * own, and moe_combine_recv needs none.
 */
int moe_dispatch_direct_noalloc(const moe_shape *shape, const uint16_t *tokens, const int32_t *topk_idx,
                                uint8_t *x_q, float *x_s, int32_t *send_pos, int32_t *exp_off, int32_t *row_src,
                                uint32_t *flags, void *stream);

/*
 * moe_dispatch_direct in a single launch, for decode-sized batches (the
 * low-latency mode of the AWS China blog "750B MoE model migration from a
 * self-built RoCE cluster to AWS EFA", section 4.4: one kernel, no host in
 * the loop).  Same arguments, results and workspace tables as
 * moe_dispatch_direct, with the limits and the exchange protocol of
 * moe_dispatch_send_ll: every rank's slots must fit one routing chunk
 * (T*k <= 4096, else MOE_EINVAL), and a wait inside the launch that gives up
 * sets MOE_FLAG_TIMEOUT and drops its rows.  tokens may be NULL (layout
 * only).
 */
int moe_dispatch_direct_ll(const moe_shape *shape, const uint16_t *tokens, const int32_t *topk_idx, uint8_t *x_q,
                           float *x_s, int32_t *send_pos, int32_t *exp_off, int32_t *row_src, void *ws,
                           void *stream);

/*
 * Dispatch, receive half ("Dispatch and combine": the receive buffer is
 * shuffled into the output tensor handed to the grouped GEMM).  Uses only
 * the exchanged counts held in ws.
 *   recv_q, recv_s  the receive regions written by moe_dispatch_send.
 *   x_q, x_s        out, same shapes: rank d's rows start at base[d] and are
 *                   expert-major.  recv_q, recv_s, x_q and x_s may all be
 *                   NULL together: then only exp_off and row_src are
 *                   produced (the layout a combine needs).
 *   exp_off         int32 [N][L+1] out: row offsets of rank d's experts,
 *                   relative to base[d] (exp_off[d][L] = rows received).
 *   row_src         int32 [rows] out: for each written expert-major row,
 *                   s*T*k + send_pos of the slot it carries (where combine
 *                   returns it); -1 for a row dropped by a fixed-region
 *                   overflow.  Rows beyond each region's count are untouched.
 */
int moe_dispatch_recv(const moe_shape *shape, const uint8_t *recv_q, const float *recv_s, const void *ws,
                      uint8_t *x_q, float *x_s, int32_t *exp_off, int32_t *row_src, void *stream);

/*
 * Combine, send half ("Dispatch and combine": rows go back to their source,
 * one contiguous run per peer, with offsets known from dispatch).
 *   y_em   bf16 [rows][H], 16-B aligned: expert outputs in the same row order
 *          as x_q (the grouped GEMM's output).
 *   row_src  as written by moe_dispatch_recv.
 *   comb   bf16 [N][T*k][H] out, 16-B aligned: comb[row_src[i]] = y_em[i].
 *          With fixed regions, the row of a valid slot that an overflow left
 *          without an expert-major row (so no row_src names it) is written
 *          as zeros, so that moe_combine_recv skips it exactly; rows at
 *          positions no valid slot has are untouched.  It may alias memory
 *          no longer needed by dispatch ("buffers are reused between
 *          dispatch and combine").
 */
int moe_combine_send(const moe_shape *shape, const uint16_t *y_em, const int32_t *row_src, const void *ws,
                     uint16_t *comb, void *stream);

/*
 * Combine, receive half ("Introduction": weighted average; "Dispatch and
 * combine": accumulate on the receive side).
 *   comb      bf16 [N][T*k][H], from moe_combine_send.
 *   send_pos  int32 [N][T][k], from moe_dispatch_send.
 *   topk_w    fp32 [N][T][k]: router weights (they sum to 1 per token, so the
 *             sum below is the weighted average; no division by sum(w)).
 *   out       bf16 [N][T][H] out, 16-B aligned:
 *             out[s][t] = bf16_rne(sum_j w[s][t][j] * comb[s*T*k + send_pos]),
 *             float32 accumulation in slot order j = 0..k-1 with no fused
 *             multiply-add; dropped slots contribute nothing.
 * Needs no workspace.
 */
int moe_combine_recv(const moe_shape *shape, const uint16_t *comb, const int32_t *send_pos, const float *topk_w,
                     uint16_t *out, void *stream);

/*
 * Combine in one pass, pulling ("Dispatch and combine": peers whose buffers
 * are mapped can pull tokens directly; on one GPU every rank is such a peer).
 * Each source rank reads its slots' rows straight out of the expert-major
 * outputs, so no combine_send copy is made:
 *   out[s][t] = bf16_rne(sum_j w[s][t][j] * y_em[row of slot (s,t,j)]),
 * the row found from the routing tables in ws (the same row moe_combine_send
 * would copy), with the same float32 arithmetic and slot order as
 * moe_combine_recv, hence the same bytes.  Slots without a row (bad id, or a
 * fixed region that overflowed) contribute nothing.
 *   y_em      bf16 [rows][H], 16-B aligned, expert-major (as for combine_send).
 *   topk_idx  int32 [N][T][k], as given to moe_dispatch_send.
 *   send_pos  int32 [N][T][k], from moe_dispatch_send.
 *   topk_w    fp32 [N][T][k].
 *   ws        the workspace of that dispatch.
 *   out       bf16 [N][T][H] out, 16-B aligned.
 */
int moe_combine_pull(const moe_shape *shape, const uint16_t *y_em, const int32_t *topk_idx, const int32_t *send_pos,
                     const float *topk_w, const void *ws, uint16_t *out, void *stream);

/*
 * Combine with send-side partial accumulation, send half ("Evaluation:
 * dispatch/combine latency": summing a token's rows on the send side of
 * combine cuts the data sent, possibly at some cost in accuracy).  A group is
 * the set of a token's slots whose expert-major rows sit on one rank; its
 * leader is its first slot.  For every group of every token (s, t):
 *   comb[s*T*k + send_pos[s][t][leader]] =
 *       bf16_rne(sum over the group's slots j, in slot order, of w[s][t][j] * y_j),
 * float32 accumulation with no fused multiply-add.  Rows of comb that no
 * group leads are left untouched.  Slots without a row (bad id, or a row a
 * full fixed region dropped) belong to no group.
 *   y_em, topk_idx, send_pos, topk_w, ws   as for moe_combine_pull (the
 *                                          weights travel with the tokens).
 *   comb   bf16 [N][T*k][H] out, 16-B aligned.
 */
int moe_combine_send_partial(const moe_shape *shape, const uint16_t *y_em, const int32_t *topk_idx,
                             const int32_t *send_pos, const float *topk_w, const void *ws, uint16_t *comb,
                             void *stream);

/*
 * Combine with send-side partial accumulation, receive half:
 *   out[s][t] = bf16_rne(sum over the token's groups, in leader order, of
 *               the group row comb[s*T*k + send_pos[s][t][leader]]),
 * float32 accumulation, no weights (the sender applied them).
 *   comb      from moe_combine_send_partial.
 *   topk_idx, send_pos, ws   as given to moe_combine_send_partial.
 *   out       bf16 [N][T][H] out, 16-B aligned.
 * It differs from moe_combine_recv by the rounding of each group sum to bf16:
 * |out - sum_j w_j y_j| <= 2^-8 (|out| + sum_g |group row g|)
 *                          + 2k 2^-24 sum_j |w_j y_j|.
 */
int moe_combine_recv_partial(const moe_shape *shape, const uint16_t *comb, const int32_t *topk_idx,
                             const int32_t *send_pos, const void *ws, uint16_t *out, void *stream);

/*
 * Wait for `stream`, return the sticky error bits accumulated in ws since the
 * last call (MOE_FLAG_*) through *flags, and clear them.  The only call that
 * blocks the host.
 */
int moe_status(void *ws, void *stream, uint32_t *flags);

/*
 * Copy the routing tables held in ws after moe_dispatch_send into caller
 * arrays (device, int32; any may be NULL): cnt [N][E], send_off [N][E+1],
 * recv_off [N(dest)][N(source)+1] (with early rows: offsets of each
 * source's rows beyond its first C, from region row N*C), recv_total [N]
 * (all rows for each destination), base [N+1] (first row of each region;
 * base[N] = rows in use when packed, N*R when fixed).
 */
int moe_layout_export(const moe_shape *shape, const void *ws, int32_t *cnt, int32_t *send_off, int32_t *recv_off,
                      int32_t *recv_total, int32_t *base, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_EP_H */
