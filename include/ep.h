/*
 * ep.h -- C ABI of the MI355X (gfx950) MoE expert-parallel dispatch / combine
 * library (libep.so).
 *
 * The operations are the expert-parallel hot path of the page
 * "[Not ready] MSCCLPP EP implementation #852" (microsoft/mscclpp pull 852):
 *   - get_dispatch_layout (PR body, "Scope / Intranode" and "Internode HT"),
 *   - dispatch and combine over the x[T,H] bf16 / topk_idx[T,k] int64 /
 *     topk_weights[T,k] fp32 tensor ABI (same section),
 *   - the low-latency dispatch with per-token FP8 casting and one scale per
 *     128 channels (low-latency port commit, dispatch<kUseFP8,...>),
 *   - combine consuming the receiver-side layout produced by dispatch (commit
 *     fixing internode HT combine: receiver-side prefix sums).
 * On one GPU every destination "rank" is a contiguous range of one receive
 * buffer in this GPU's HBM: experts are split into num_ranks contiguous
 * blocks of num_experts/num_ranks, and rank r's rows are
 * [recv_rank_offset[r], recv_rank_offset[r+1]).
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * Pointers.  Every array argument is a DEVICE pointer (HBM of the current HIP
 * device), row-major and densely packed, owned by the caller; the library
 * keeps no reference after the call returns and allocates nothing at run
 * time (ep_dispatch_noalloc's fixed scratch is part of the loaded code).  The
 * workspace is caller-owned device memory of at least the size reported by
 * the matching *_workspace_bytes() call, 4-byte aligned (the kernels keep
 * 32-bit counters there; EP_ERR_INVALID_ARGUMENT otherwise); its contents on
 * entry do not matter and on exit are unspecified.
 *
 * bf16 data is passed as raw 16-bit patterns (void*).
 *
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Every call
 * only validates its arguments on the host and enqueues kernels on `stream`;
 * it never synchronises.  Outputs are valid once the stream reaches that
 * point.  Calls on different streams touching disjoint buffers may run
 * concurrently; the library holds no mutable global state apart from the
 * fixed device scratch of ep_dispatch_noalloc (below) and the per-device
 * cache of its address, filled once under a lock.
 *
 * Routing slots.  Slot (t, j) is valid iff 0 <= topk_idx[t*k + j] <
 * num_experts.  Any other value (conventionally -1) is an empty slot: it gets
 * no receive row, no count, and token_row = -1.  The same expert may appear
 * twice in a token; each slot then gets its own row.
 *
 * Receive order.  Rows are grouped by expert (ascending), so every rank's
 * experts are one contiguous range; inside an expert, rows follow (t, j)
 * ascending.  This order is unique, so every index output is deterministic
 * and bit-reproducible.  Receive buffers are sized at capacity
 * num_tokens * num_topk rows; the filled row count is
 * recv_expert_offset[num_experts]; rows beyond it are not written.
 *
 * Errors.  Every entry point returns an ep_status_t (as int).  Invalid
 * arguments are detected on the host before anything is enqueued and leave
 * all outputs untouched.  EP_ERR_HIP reports a failed launch
 * (hipGetLastError).  ep_last_error() returns a thread-local description of
 * the last failure on the calling thread.  No C++ exception crosses the ABI.
 */
#ifndef EP_MI355X_EP_H
#define EP_MI355X_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EP_OK = 0,
    EP_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, misalignment, ... */
    EP_ERR_UNSUPPORTED = 2,        /* valid but beyond the library's limits     */
    EP_ERR_WORKSPACE_TOO_SMALL = 3,
    EP_ERR_HIP = 4                 /* a HIP runtime call or launch failed        */
} ep_status_t;

/* Limits of the library (EP_ERR_UNSUPPORTED beyond them). */
#define EP_MAX_TOPK 64          /* num_topk                                   */
#define EP_MAX_RANKS 64         /* num_ranks                                  */
#define EP_MAX_EXPERTS 2048     /* num_experts                                */
/* The bf16 copies (ep_dispatch, ep_dispatch_cached, ep_dispatch_ht,
 * ep_dispatch_ll) run in one
 * launch of T * ceil(H / 1024) blocks of 64 * min(fanout, 8) threads, where
 * fanout is num_topk (num_ranks for ep_dispatch_ht); a launch holds at most
 * 2^32 - 1 threads, and larger shapes return EP_ERR_UNSUPPORTED before any
 * work is enqueued (e.g. T = 2^20 tokens of H = 8192 at fanout 8). */

/* Static description of a status code; never NULL. */
const char* ep_status_string(int status);

/* Thread-local text of the last non-EP_OK status returned on this thread. */
const char* ep_last_error(void);

/* Library version string, e.g. "ep-mi355x 0.1 gfx950". */
const char* ep_version(void);

/* ---------------------------------------------------------------------------
 * ep_get_dispatch_layout -- routing histogram of one batch (get_dispatch_layout
 * of the page's "Scope / Intranode"; the per-group count is the per-RDMA-rank
 * count of "Scope / Internode HT", a group being ranks_per_group consecutive
 * ranks).
 *
 *   topk_idx              [T, k] int64   routing (see "Routing slots")
 *   num_tokens_per_rank   [R]    int32   out: tokens with >= 1 valid slot on r
 *   num_tokens_per_group  [R/P]  int32   out: tokens touching any rank of group
 *                                        g (may be NULL)
 *   num_tokens_per_expert [E]    int32   out: valid slots routed to e
 *   is_token_in_rank      [T, R] uint8   out: 1 iff token t has a valid slot on
 *                                        rank r, else 0
 *
 * Requires T >= 0, 1 <= k <= EP_MAX_TOPK, 1 <= R <= EP_MAX_RANKS,
 * E % R == 0, E <= EP_MAX_EXPERTS, 1 <= P, R % P == 0.  T == 0 writes zero
 * counts.  Workspace: ep_layout_workspace_bytes(T, E, R, P).
 * ------------------------------------------------------------------------- */
size_t ep_layout_workspace_bytes(int64_t num_tokens, int num_experts, int num_ranks,
                                 int ranks_per_group);

int ep_get_dispatch_layout(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                           int num_experts, int num_ranks, int ranks_per_group,
                           int32_t* num_tokens_per_rank, int32_t* num_tokens_per_group,
                           int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ep_dispatch -- permute each token's hidden vector into the contiguous
 * per-rank / per-expert receive buffer (intranode dispatch of "Scope /
 * Intranode"), and emit the receiver-side maps that combine consumes.
 *
 *   x                  [T, H]  bf16  in: token activations (16-byte aligned)
 *   topk_idx           [T, k]  int64 in
 *   topk_weights       [T, k]  fp32  in (may be NULL)
 *   recv_x             [T*k, H] bf16 out: recv_x[token_row[t,j]] = x[t], bit
 *                                    for bit (16-byte aligned)
 *   recv_src_idx       [T*k]   int32 out: source token of each filled row
 *   recv_topk_weights  [T*k]   fp32  out: topk_weights[t,j] of each filled row
 *                                    (may be NULL; ignored if topk_weights is)
 *   recv_expert_offset [E+1]   int32 out: first row of each expert; [E] = rows
 *   recv_rank_offset   [R+1]   int32 out: recv_expert_offset[r*E/R] (may be NULL)
 *   token_row          [T, k]  int32 out: row of slot (t,j), -1 if empty
 *
 * Requires H % 8 == 0 (rows are whole 16-byte vectors), T*k < 2^31, the
 * layout limits above and (bf16) the copy-launch limit.
 * Workspace: ep_dispatch_workspace_bytes(T, k, E).
 * The offsets are computed from topk_idx itself, so no earlier call's output
 * is trusted and every write stays inside the buffers described above.
 * ------------------------------------------------------------------------- */
size_t ep_dispatch_workspace_bytes(int64_t num_tokens, int num_topk, int num_experts);

int ep_dispatch(const void* x, const int64_t* topk_idx, const float* topk_weights,
                int64_t num_tokens, int hidden, int num_topk, int num_experts, int num_ranks,
                void* recv_x, int32_t* recv_src_idx, float* recv_topk_weights,
                int32_t* recv_expert_offset, int32_t* recv_rank_offset, int32_t* token_row,
                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ep_dispatch_noalloc -- ep_dispatch for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same operation, kernels and outputs as ep_dispatch,
 * with no workspace argument.  The receive-order scratch is a fixed device
 * array inside the library, EP_NOALLOC_SCRATCH_BYTES per GPU, held until the
 * process ends; the call itself allocates nothing.
 *
 * Arguments and outputs as ep_dispatch.  The stream must belong to the
 * current HIP device.  A batch whose scratch need,
 * ep_dispatch_workspace_bytes(T, k, E), exceeds EP_NOALLOC_SCRATCH_BYTES
 * returns EP_ERR_UNSUPPORTED before anything is enqueued (e.g. 32768 tokens
 * at top-8 need 64 KiB + 256 B over 256 experts, 512 KiB + 256 B over 2048).
 * All calls on one GPU share that GPU's array: calls that overlap on one GPU
 * (two streams, two threads) race and must be serialised by the caller.
 * ------------------------------------------------------------------------- */
#define EP_NOALLOC_SCRATCH_BYTES (1u << 20)

int ep_dispatch_noalloc(const void* x, const int64_t* topk_idx, const float* topk_weights,
                        int64_t num_tokens, int hidden, int num_topk, int num_experts,
                        int num_ranks, void* recv_x, int32_t* recv_src_idx,
                        float* recv_topk_weights, int32_t* recv_expert_offset,
                        int32_t* recv_rank_offset, int32_t* token_row, void* stream);

/* ---------------------------------------------------------------------------
 * ep_dispatch_fp8 -- ep_dispatch with the low-latency FP8 cast (low-latency
 * port commit, dispatch<kUseFP8,...>).  For token t and 128-channel block c:
 *   a = max |x[t, 128c .. 128c+127]|,  s = a / 448 (IEEE fp32 division),
 *   code = E4M3(x / s) (OCP E4M3FN, round to nearest even, saturating at
 *   +-448), or 0x00 for every channel when s == 0.
 * Every row of the token receives the same codes and scales:
 *   recv_x_fp8  [T*k, H]     uint8 out: E4M3FN codes (16-byte aligned)
 *   recv_scales [T*k, H/128] fp32  out: s per 128-channel block
 * All other arguments as ep_dispatch.  Requires H % 128 == 0.
 * Workspace: ep_dispatch_workspace_bytes(T, k, E).
 * ------------------------------------------------------------------------- */
int ep_dispatch_fp8(const void* x, const int64_t* topk_idx, const float* topk_weights,
                    int64_t num_tokens, int hidden, int num_topk, int num_experts,
                    int num_ranks, uint8_t* recv_x_fp8, float* recv_scales,
                    int32_t* recv_src_idx, float* recv_topk_weights,
                    int32_t* recv_expert_offset, int32_t* recv_rank_offset,
                    int32_t* token_row, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ---------------------------------------------------------------------------
 * ep_dispatch_cached / ep_dispatch_fp8_cached -- repeat dispatch that reuses
 * the receive map of an earlier ep_dispatch / ep_dispatch_fp8 with the same
 * routing (the cached_notify of page #852, "Scope / Internode HT": a repeat
 * dispatch skips the layout and count exchange).  No receive-order work is
 * done: for every slot (t, j) whose row r = token_row[t, j] lies in
 * [0, recv_rows), row r receives x[t] (bf16, bit for bit) or its FP8 cast
 * (codes and scales exactly as ep_dispatch_fp8 computes them).  Slots with
 * any other row, including -1, are skipped, so no map can make the kernel
 * write outside the recv_rows rows given.  Other rows are not written.
 *
 *   x           [T, H]          bf16  in (16-byte aligned)
 *   token_row   [T, k]          int32 in (an earlier dispatch's output)
 *   recv_x      [recv_rows, H]  bf16  out (16-byte aligned)
 *   recv_x_fp8  [recv_rows, H]  uint8 out (16-byte aligned), recv_scales
 *               [recv_rows, H/128] fp32 out (FP8 variant)
 * Requires H % 8 == 0 (bf16) or H % 128 == 0 (FP8), 1 <= k <= EP_MAX_TOPK
 * and (bf16) the copy-launch limit.
 * No workspace.  T == 0 or recv_rows == 0 enqueues nothing.
 * ------------------------------------------------------------------------- */
int ep_dispatch_cached(const void* x, const int32_t* token_row, int64_t num_tokens, int hidden,
                       int num_topk, void* recv_x, int64_t recv_rows, void* stream);

int ep_dispatch_fp8_cached(const void* x, const int32_t* token_row, int64_t num_tokens,
                           int hidden, int num_topk, uint8_t* recv_x_fp8, float* recv_scales,
                           int64_t recv_rows, void* stream);

/* ---------------------------------------------------------------------------
 * ep_dispatch_ht -- rank-deduplicated ("high-throughput") dispatch: the
 * intranode dispatch of page #852, "Scope / Intranode", which sends each
 * token once to every rank hosting at least one of its experts, the receiver
 * seeing the token's top-k ids remapped to its local experts.  One receive
 * row per (token t, rank r) with t routed to r (is_token_in_rank[t, r] = 1),
 * ordered by rank, then token:
 *
 *   recv_x            [T*R, H]  bf16  out: row = x[t], bit for bit (capacity
 *                                     T*R rows; recv_rank_offset[R] filled)
 *   recv_src_idx      [T*R]     int32 out: source token of each filled row
 *   recv_topk_idx     [T*R, k]  int64 out: topk_idx[t, j] - r*E/R when that
 *                                     expert is on rank r, else -1
 *   recv_topk_weights [T*R, k]  fp32  out: topk_weights[t, j] on the same
 *                                     condition, else 0 (may be NULL)
 *   recv_rank_offset  [R+1]     int32 out: first row of each rank; [R] = rows
 *   token_rank_row    [T, R]    int32 out: row of (t, r), or -1
 *
 * The matching combine is ep_combine(expert_out, rows, token_rank_row, NULL,
 * T, H, R, out): out[t] = bf16(sum over ranks, in rank order, of the rank's
 * row for t), each row holding that rank's already weighted partial result.
 * Requires H % 8 == 0, T*R < 2^31, the routing limits above and the
 * copy-launch limit with fanout R.
 * Workspace: ep_dispatch_ht_workspace_bytes(T, R).
 * ------------------------------------------------------------------------- */
size_t ep_dispatch_ht_workspace_bytes(int64_t num_tokens, int num_ranks);

int ep_dispatch_ht(const void* x, const int64_t* topk_idx, const float* topk_weights,
                   int64_t num_tokens, int hidden, int num_topk, int num_experts, int num_ranks,
                   void* recv_x, int32_t* recv_src_idx, int64_t* recv_topk_idx,
                   float* recv_topk_weights, int32_t* recv_rank_offset, int32_t* token_rank_row,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ep_dispatch_ll / ep_dispatch_ll_fp8 -- padded expert-major ("low-latency")
 * dispatch.  Page #852: the LL benchmark's receive buffer is one fixed-size
 * region per expert (the commit that stops cloning that buffer inside the
 * timed loop), and the low-latency runtime is tested at capacities 1 and 2.
 * With one source the receive buffer is [E, capacity, H]; expert e owns rows
 * e*capacity .. e*capacity + capacity - 1, filled in (token, slot) order, and
 * a slot that finds its region full is dropped:
 *
 *   recv_x            [E, capacity, H]  bf16 out: slot = x[t], bit for bit
 *     (ep_dispatch_ll_fp8: recv_x_fp8 [E, capacity, H] E4M3FN codes and
 *      recv_scales [E, capacity, H/128] fp32, the cast of ep_dispatch_fp8)
 *   recv_count        [E]          int32 out: min(slots routed to e, capacity)
 *   recv_src_idx      [E, capacity] int32 out: source token of each filled slot
 *   recv_topk_weights [E, capacity] fp32  out: topk_weights[t, j] of each
 *                                     filled slot (may be NULL; ignored if
 *                                     topk_weights is NULL)
 *   token_slot        [T, k]       int32 out: e*capacity + position of (t, j),
 *                                     or -1 (empty slot, or dropped)
 *
 * Rows recv_count[e] .. capacity-1 of each expert are not written.  Combine:
 * ep_combine(expert_out [E*capacity, H], E*capacity, token_slot, weights, ...);
 * a dropped slot then contributes nothing.  capacity = T never drops.
 * Requires 1 <= capacity, E*capacity < 2^31, H % 8 == 0 (bf16) or
 * H % 128 == 0 (FP8), the routing limits above (ranks are not involved) and
 * (bf16) the copy-launch limit.  Workspace: ep_dispatch_ll_workspace_bytes.
 * ------------------------------------------------------------------------- */
size_t ep_dispatch_ll_workspace_bytes(int64_t num_tokens, int num_topk, int num_experts);

int ep_dispatch_ll(const void* x, const int64_t* topk_idx, const float* topk_weights,
                   int64_t num_tokens, int hidden, int num_topk, int num_experts, int capacity,
                   void* recv_x, int32_t* recv_count, int32_t* recv_src_idx,
                   float* recv_topk_weights, int32_t* token_slot, void* workspace,
                   size_t workspace_bytes, void* stream);

int ep_dispatch_ll_fp8(const void* x, const int64_t* topk_idx, const float* topk_weights,
                       int64_t num_tokens, int hidden, int num_topk, int num_experts,
                       int capacity, uint8_t* recv_x_fp8, float* recv_scales,
                       int32_t* recv_count, int32_t* recv_src_idx, float* recv_topk_weights,
                       int32_t* token_slot, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ---------------------------------------------------------------------------
 * ep_combine -- gather each token's expert outputs back and sum them weighted
 * by topk_weights (intranode combine of "Scope / Intranode", consuming the
 * receiver-side map token_row that dispatch produced).  For every t, h:
 *   acc = +0.0f;  for j = 0 .. k-1 in this order, if 0 <= token_row[t,j] < num_rows:
 *       acc = fmaf(topk_weights[t,j], expert_out[token_row[t,j], h], acc);
 *   combined_x[t, h] = bf16(acc), rounded to nearest even.
 * topk_weights may be NULL: every weight is then 1 (a plain fp32 sum in j
 * order), which is the combine of ep_dispatch_ht's per-rank rows.
 *
 *   expert_out   [num_rows, H] bf16 in (16-byte aligned)
 *   token_row    [T, k]        int32 in (from ep_dispatch; a slot whose row
 *                              lies outside [0, num_rows) contributes nothing.
 *                              For small batches the kernel still issues a
 *                              load for such a slot -- of row 0 of expert_out,
 *                              or, when num_rows == 0, of the token's own
 *                              combined_x segment before writing it -- and
 *                              discards the value; nothing outside the
 *                              buffers described here is read)
 *   topk_weights [T, k]        fp32  in (NULL: all weights 1)
 *   combined_x   [T, H]        bf16  out (16-byte aligned)
 * Requires H % 8 == 0, 1 <= k <= EP_MAX_TOPK, num_rows >= 0.  No workspace.
 * ------------------------------------------------------------------------- */
int ep_combine(const void* expert_out, int64_t num_rows, const int32_t* token_row,
               const float* topk_weights, int64_t num_tokens, int hidden, int num_topk,
               void* combined_x, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_MI355X_EP_H */
