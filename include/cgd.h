/*
 * cgd.h - C ABI of libcgd: the MoE expert-parallel layout / dispatch / combine
 * hot path on one AMD MI355X (gfx950).
 *
 * The operations follow the DeepEP-style expert-parallel layer described by:
 *   - the get_dispatch_layout API page (sgl-kernel-npu deep_ep docs),
 *     sections "Parameters", "Return Values" and "Notes";
 *   - the DeepEP Python interface notes ("4 Python接口"), section "Dispatch API"
 *     (inputs, outputs, cached mode, expert_alignment, async/event handling);
 *   - the DeepEP legacy test analysis page: layout cross-check excerpt,
 *     low-latency per-expert check (expert id = rank * num_local_experts + i),
 *     low-latency combine check (x scaled by the sum of unmasked weights),
 *     and the handle layouts of the legacy.py excerpts.
 *
 * The "ranks" are logical partitions of the expert set inside one device:
 * rank r owns experts [r*L, (r+1)*L) with L = num_experts / num_ranks.
 *
 * Conventions for every call:
 *   - Every pointer argument is a DEVICE pointer, except where noted. The
 *     caller allocates and frees all memory, including workspaces; the library
 *     never allocates device memory and never synchronises the stream.
 *   - Every call only enqueues kernels on `stream` and returns (the pages'
 *     async_finish=True). The caller orders work with its own events
 *     (hipEventRecord / hipStreamWaitEvent), which replaces the pages'
 *     previous_event / EventOverlap objects. Inputs must stay alive and
 *     unmodified until the stream has passed the call.
 *   - Pointers to bf16 rows and the is_token_in_rank output must be 16-byte
 *     aligned; other pointers must be aligned to their element type.
 *   - bf16 data are IEEE bfloat16 bit patterns (uint16 storage).
 *   - Return value: CGD_OK, or a negative cgd_status; then nothing was
 *     enqueued (except for CGD_ERR_HIP, where a launch failed) and
 *     cgd_last_error() returns a message for the calling thread.
 *   - Argument limits mirror the get_dispatch_layout API page: num_topk in
 *     [1,16], num_experts in [1,512], num_ranks in [1,384], num_experts a
 *     multiple of num_ranks. num_tokens may be 0 (a documented extension:
 *     all counts are then zero). hidden must be a positive multiple of 8.
 *   - Device-side data preconditions are not checked on the host: topk_idx
 *     entries are expected in [-1, num_experts). A value outside that range
 *     is treated as -1 (not selected) by every kernel, so it never causes an
 *     out-of-bounds access. The pages' routing never repeats an expert within
 *     a token; if a row does, every selected slot still gets a row of its
 *     own, in ascending (token, slot) order like any other, and the token
 *     counts once per rank in the layout.
 */
#ifndef CGD_H
#define CGD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CGD_OK = 0,
    CGD_ERR_INVALID_ARG = -1, /* a size, pointer or alignment is invalid */
    CGD_ERR_CAPACITY = -2,    /* recv_capacity is below cgd_dispatch_capacity() */
    CGD_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
    CGD_ERR_HIP = -4          /* a HIP launch failed */
} cgd_status;

/* Library version string (host pointer, static storage). */
const char* cgd_version(void);

/* Loads libcgd's GPU code on the calling thread's current device ahead of
 * use (the first-call latency page: a process's first dispatch is far slower
 * than later ones, part of it one-time loading). The runtime otherwise loads
 * each of libcgd's code objects on the first launch of one of its kernels,
 * inside that first call. Host only: allocates nothing, enqueues nothing.
 * Optional; call once per device. Returns CGD_ERR_HIP if the code cannot be
 * loaded on this device. */
int cgd_init(void);

/* Message for the last non-OK status returned on the calling thread
 * (host pointer, valid until the next call on that thread). */
const char* cgd_last_error(void);

/* Workspace bytes cgd_get_dispatch_layout needs for these sizes (host only;
 * 0 if the sizes are invalid). The workspace must be zero-filled before its
 * first use; every completed call leaves the words that must start at zero
 * (here one count accumulator per expert and rank; in the other workspaces a
 * ticket at their start) zero again, and everything else in it is rewritten
 * before it is read, so one workspace serves any number of calls, of any
 * sizes, that are ordered on one stream. Calls that may run concurrently
 * need separate workspaces. */
size_t cgd_layout_workspace_bytes(int64_t num_tokens, int num_topk, int num_experts, int num_ranks);

/* Workspace bytes cgd_dispatch, cgd_dispatch_plan and their layout-fused
 * forms need for these sizes (host only; 0 if invalid). Same zero-fill and
 * reuse rules as the layout workspace. num_ranks sizes the per-rank partial
 * counts of the layout-fused forms. */
size_t cgd_dispatch_workspace_bytes(int64_t num_tokens, int num_topk, int num_experts, int num_ranks);

/* Rows a receive buffer needs for ANY routing of these sizes (host only):
 * num_tokens * num_topk + num_experts * (expert_alignment - 1), or -1 if the
 * sizes are invalid or the result exceeds INT32_MAX. Knowing this on the host
 * means no device-to-host copy is needed before dispatch, the purpose of the
 * pages' num_worst_tokens argument (Python interface notes, "Dispatch API"). */
int64_t cgd_dispatch_capacity(int64_t num_tokens, int num_topk, int num_experts, int expert_alignment);

/* get_dispatch_layout (get_dispatch_layout API page, "Return Values"):
 *   topk_idx               int64 [num_tokens, num_topk], row-major; -1 = not selected
 *   num_tokens_per_rank    int32 [num_ranks]   out: distinct tokens with >= 1 expert on the rank
 *   num_tokens_per_expert  int32 [num_experts] out: selected slots per expert
 *   is_token_in_rank       uint8 [num_tokens, num_ranks] row-major, out: 1 if the token
 *                          selects an expert of the rank, else 0 (torch.bool storage)
 *   workspace              >= cgd_layout_workspace_bytes(...) bytes, see above
 * The pages' num_tokens_per_rdma_rank output is not produced (it is None for a
 * single node). Outputs are fully overwritten. */
int cgd_get_dispatch_layout(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                            int num_ranks, int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                            uint8_t* is_token_in_rank, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Dispatch (Python interface notes, "Dispatch API", non-cached mode):
 * places every selected (token, slot) pair in a contiguous receive segment of
 * its expert and copies the token's bf16 row there.
 *   x                  bf16 [num_tokens, hidden]
 *   topk_idx           int64 [num_tokens, num_topk]; -1 = not selected
 *   expert_alignment   >= 1; each expert's segment size is its row count
 *                      rounded up to a multiple of this value
 *   recv_x             bf16 [recv_capacity, hidden] out: row dst_row[t,k] = x[t], bit for bit;
 *                      alignment-padding rows and rows past the data are not written
 *   recv_capacity      rows of recv_x and recv_src_idx; >= cgd_dispatch_capacity(...)
 *   expert_offset      int32 [num_experts + 1] out: segment e is rows
 *                      [expert_offset[e], expert_offset[e+1]); segments are in
 *                      ascending expert id, hence grouped by rank
 *   num_recv_tokens_per_expert
 *                      int32 [num_experts] out, or NULL (not written): the aligned
 *                      segment sizes, each expert's row count rounded up to
 *                      expert_alignment (the dispatch output of that name in the
 *                      "Dispatch API" section); equal to expert_offset[e+1] - expert_offset[e]
 *   recv_src_idx       int32 [recv_capacity] out: source token of each data row, -1 elsewhere
 *   dst_row            int32 [num_tokens, num_topk] out: receive row of each slot, -1 if
 *                      not selected. Inside a segment rows follow ascending (token, slot)
 *   workspace          >= cgd_dispatch_workspace_bytes(...) bytes
 * (expert_offset, recv_src_idx, dst_row) is the handle for cached dispatch and
 * for combine. Counts are derived from topk_idx itself, so the layout's
 * num_tokens_per_expert is not an input here and cannot disagree with the
 * routing (on one GPU no count exchange precedes the data). */
int cgd_dispatch(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx, int num_topk,
                 int num_experts, int num_ranks, int expert_alignment, void* recv_x, int64_t recv_capacity,
                 int32_t* expert_offset, int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* dst_row,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Dispatch in two steps on one stream: cgd_dispatch is exactly
 * cgd_dispatch_plan followed by cgd_dispatch_cached with the plan's dst_row
 * and the same capacity. The plan needs only the routing, like the notify
 * stage that precedes data movement in the pages' dispatch (the
 * diagnostic-probes PR page, "Implementation": notify kernels before the
 * dispatch data kernels; the first-call latency blog page: tensor sizes are
 * notified in advance), so a caller may enqueue it early; it writes the whole
 * handle (expert_offset, recv_src_idx, dst_row, as cgd_dispatch describes)
 * and num_recv_tokens_per_expert, and the row copy that follows moves data
 * only. Batches of one 256-token
 * tile are planned in one launch, larger ones in two (per-tile ranks, then
 * final rows). Arguments and errors as cgd_dispatch; the workspace is not
 * needed once the plan has run. */
int cgd_dispatch_plan(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts, int num_ranks,
                      int expert_alignment, int64_t recv_capacity, int32_t* expert_offset,
                      int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* dst_row, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* cgd_get_dispatch_layout and cgd_dispatch_plan in one call: both read the
 * same routing, so one pass over each 256-token tile (one launch, plus the
 * final-row launch of a batch of several tiles) produces the layout outputs
 * (as cgd_get_dispatch_layout, same arguments and rules; no layout workspace
 * is needed) and the dispatch handle (as cgd_dispatch_plan). */
int cgd_layout_and_dispatch_plan(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                                 int num_ranks, int expert_alignment, int64_t recv_capacity,
                                 int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                                 uint8_t* is_token_in_rank, int32_t* expert_offset,
                                 int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* dst_row,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* cgd_get_dispatch_layout and cgd_dispatch in one call: the layout outputs
 * (as cgd_get_dispatch_layout; no layout workspace is needed) and the
 * dispatch (as cgd_dispatch: handle and rows), same arguments and rules.
 * A batch of at most 256 tokens takes one launch (layout, plan and rows, the
 * decode case); larger ones are cgd_layout_and_dispatch_plan followed by
 * cgd_dispatch_cached. */
int cgd_layout_and_dispatch(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx, int num_topk,
                            int num_experts, int num_ranks, int expert_alignment, void* recv_x,
                            int64_t recv_capacity, int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                            uint8_t* is_token_in_rank, int32_t* expert_offset, int32_t* num_recv_tokens_per_expert,
                            int32_t* recv_src_idx, int32_t* dst_row, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* cgd_layout_and_dispatch for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, outputs and errors without the workspace,
 * which is a file-scope device array inside the library instead; the call
 * allocates nothing (no hipMalloc, no library allocation). The caller still
 * passes every input and output.
 *   Limit: sizes whose workspace (cgd_dispatch_workspace_bytes) exceeds
 *   8 MiB are rejected with CGD_ERR_WORKSPACE before anything is enqueued
 *   (about 1.9 million selected slots, num_tokens * num_topk).
 *   Each GPU the library runs on holds its own 8 MiB copy of the array until
 *   the process ends. Every call on a GPU shares that GPU's copy: calls that
 *   overlap on one GPU (different streams, or graphs replayed concurrently)
 *   race and must be ordered by the caller. The first call on a device looks
 *   up the array's address there and enqueues, before its own work, one
 *   one-wave kernel that clears the words that must start at zero; every
 *   call leaves them zero again. */
int cgd_layout_and_dispatch_noalloc(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                    int num_topk, int num_experts, int num_ranks, int expert_alignment, void* recv_x,
                                    int64_t recv_capacity, int32_t* num_tokens_per_rank,
                                    int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank, int32_t* expert_offset,
                                    int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* dst_row,
                                    hipStream_t stream);

/* Cached dispatch (Python interface notes, "Dispatch API", handle reuse):
 * copies rows with a dst_row from an earlier cgd_dispatch or
 * cgd_dispatch_plan, skipping the layout work. recv_x[dst_row[t,k]] = x[t]
 * for every dst_row[t,k] in [0, recv_capacity); other entries are skipped.
 * It is also the second step of a planned dispatch. */
int cgd_dispatch_cached(const void* x, int64_t num_tokens, int hidden, int num_topk, const int32_t* dst_row,
                        void* recv_x, int64_t recv_capacity, hipStream_t stream);

/* Combine (legacy test analysis page, low-latency combine check):
 *   combined_x[t] = bf16( sum over k with dst_row[t,k] >= 0, ascending k, of
 *                         topk_weights[t,k] * expert_out[dst_row[t,k]] )
 * accumulated in fp32 with fused multiply-add from +0 and rounded to nearest
 * even. A token with no selected slot gives +0.
 *   expert_out     bf16 [recv_capacity, hidden]
 *   dst_row        int32 [num_tokens, num_topk] from cgd_dispatch; entries outside
 *                  [-1, recv_capacity) are treated as -1
 *   topk_weights   fp32 [num_tokens, num_topk]
 *   combined_x     bf16 [num_tokens, hidden] out */
int cgd_combine(const void* expert_out, int64_t recv_capacity, int hidden, const int32_t* dst_row,
                const float* topk_weights, int64_t num_tokens, int num_topk, void* combined_x,
                hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Rank-granular ("normal mode") dispatch and combine.
 *
 * A token is received once by every rank that is_token_in_rank flags for it,
 * rather than once per selected expert (DeepEP legacy test analysis page:
 * normal-mode dispatch call with the layout tensors, check_data walking the
 * per-rank receive prefix sums, normal-mode combine check dividing
 * combined_x - bias_0 - bias_1 by is_token_in_rank.sum(1); DeepEP Python
 * interface notes, "Dispatch API": recv_topk_idx, recv_topk_weights and the
 * aligned per-expert receive counts). Rank r's rows are
 * [rank_offset[r], rank_offset[r+1]), ranks in order, rows inside a rank in
 * ascending token order.
 * ------------------------------------------------------------------------- */

/* Workspace bytes cgd_normal_dispatch needs (host only; 0 if invalid). Same
 * zero-fill and reuse rules as the layout workspace. */
size_t cgd_normal_workspace_bytes(int64_t num_tokens, int num_ranks);

/* Rows a rank-granular receive buffer needs for ANY routing of these sizes
 * (host only): num_tokens * min(num_topk, num_ranks), since a token reaches at
 * most that many ranks; -1 if invalid or above INT32_MAX. */
int64_t cgd_normal_capacity(int64_t num_tokens, int num_topk, int num_ranks);

/* Normal-mode dispatch (Python interface notes, "Dispatch API", non-cached
 * mode, with the layout outputs as inputs):
 *   x                      bf16 [num_tokens, hidden]
 *   is_token_in_rank       uint8 [num_tokens, num_ranks] (torch.bool storage), from
 *                          cgd_get_dispatch_layout; a row may flag at most num_topk ranks
 *   num_tokens_per_expert  int32 [num_experts] from the layout, or NULL
 *   topk_idx, topk_weights int64 / fp32 [num_tokens, num_topk], or both NULL (dispatch
 *                          without top-k: then recv_topk_idx / recv_topk_weights are NULL too;
 *                          with num_tokens = 0 they may be NULL either way)
 *   recv_x                 bf16 [recv_capacity, hidden] out: row send_row[t,r] = x[t]; rows
 *                          past the data are not written
 *   recv_capacity          >= cgd_normal_capacity(...)
 *   rank_offset            int32 [num_ranks + 1] out
 *   recv_src_idx           int32 [recv_capacity] out: source token of each row, -1 past the data
 *   send_row               int32 [num_tokens, num_ranks] out: the token's row on each rank, -1
 *                          where not flagged (the analogue of the pages' send_head)
 *   recv_topk_idx          int64 [recv_capacity, num_topk] out: slot k of a row on rank r holds
 *                          e - r*L when the token's expert e lives on rank r, else -1; -1 past the data
 *   recv_topk_weights      fp32 [recv_capacity, num_topk] out: the slot's weight where
 *                          recv_topk_idx is kept, else 0
 *   num_recv_tokens_per_expert int32 [num_experts] out (iff num_tokens_per_expert): counts
 *                          rounded up to expert_alignment (alignment only affects these counts)
 * (rank_offset, recv_src_idx, send_row) is the handle for cached dispatch and combine.
 * A malformed is_token_in_rank (more than num_topk flags in a row) never
 * causes an access outside the buffers: rows at or past recv_capacity are
 * dropped (send_row -1). */
int cgd_normal_dispatch(const void* x, int64_t num_tokens, int hidden, const uint8_t* is_token_in_rank,
                        const int32_t* num_tokens_per_expert, const int64_t* topk_idx, const float* topk_weights,
                        int num_topk, int num_experts, int num_ranks, int expert_alignment, void* recv_x,
                        int64_t recv_capacity, int32_t* rank_offset, int32_t* recv_src_idx, int32_t* send_row,
                        int64_t* recv_topk_idx, float* recv_topk_weights, int32_t* num_recv_tokens_per_expert,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Normal-mode dispatch in two steps on one stream: cgd_normal_dispatch is
 * exactly cgd_normal_dispatch_plan followed by cgd_normal_dispatch_apply with
 * the same sizes, workspace and outputs (the notify stage before the data
 * stage, as for cgd_dispatch_plan / cgd_dispatch_apply).
 *   cgd_normal_dispatch_plan   reads is_token_in_rank (and num_tokens_per_expert),
 *                              writes rank_offset (and num_recv_tokens_per_expert)
 *                              and each token's place in the workspace.
 *   cgd_normal_dispatch_apply  writes send_row, recv_src_idx, recv_topk_idx,
 *                              recv_topk_weights and copies rows.
 * Between the two calls the workspace and rank_offset must not be modified or
 * used by another call. Mismatched arguments give wrong rows but never an
 * access outside the given buffers. */
int cgd_normal_dispatch_plan(const uint8_t* is_token_in_rank, int64_t num_tokens, int num_ranks,
                             const int32_t* num_tokens_per_expert, int num_experts, int expert_alignment,
                             int32_t* rank_offset, int32_t* num_recv_tokens_per_expert, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

int cgd_normal_dispatch_apply(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                              const float* topk_weights, int num_topk, int num_experts, int num_ranks, void* recv_x,
                              int64_t recv_capacity, const int32_t* rank_offset, int32_t* recv_src_idx,
                              int32_t* send_row, int64_t* recv_topk_idx, float* recv_topk_weights,
                              const void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Cached normal-mode dispatch (handle reuse): recv_x[send_row[t,r]] = x[t] for
 * every send_row entry in [0, recv_capacity); other entries are skipped. */
int cgd_normal_dispatch_cached(const void* x, int64_t num_tokens, int hidden, int num_ranks, const int32_t* send_row,
                               void* recv_x, int64_t recv_capacity, hipStream_t stream);

/* Normal-mode combine (legacy test analysis page, normal-mode combine call and
 * check):
 *   combined_x[t] = bf16( sum over r ascending with send_row[t,r] >= 0 of
 *                         expert_out[send_row[t,r]]  + bias_0[t] + bias_1[t] )
 * summed in fp32 from +0 in that order, rounded once to nearest even.
 *   expert_out             bf16 [recv_rows, hidden]; send_row entries outside [-1, recv_rows)
 *                          are treated as -1
 *   recv_topk_weights      fp32 [recv_rows, num_topk] or NULL
 *   bias_0, bias_1         bf16 [num_tokens, hidden] each, or NULL (no term)
 *   combined_topk_weights  fp32 [num_tokens, num_topk] out (iff recv_topk_weights): sum over
 *                          the token's rows, ascending rank, of recv_topk_weights[row, k] */
int cgd_normal_combine(const void* expert_out, int64_t recv_rows, int hidden, const int32_t* send_row,
                       int64_t num_tokens, int num_ranks, const float* recv_topk_weights, int num_topk,
                       const void* bias_0, const void* bias_1, void* combined_x, float* combined_topk_weights,
                       hipStream_t stream);

/* ---------------------------------------------------------------------------
 * FP8 payload (OCP e4m3fn codes with one scale per token and 128 channels).
 *
 * The pages' FP8 form of x and recv_x is the tuple (x_e4m3 [T, H],
 * x_scales [T, H/128] fp32) with H divisible by 128 (Python interface notes,
 * "Dispatch API"); the scales may be stored column-major and the cast helpers
 * are per_token_cast_to_fp8 / per_token_cast_back (legacy test analysis page,
 * test data excerpt); the low-latency dispatch adds round_scale and use_ue8m0.
 * For each token and block of 128 channels, amax = max |x| floored at 1e-4:
 *   CGD_SCALE_F32    scale = amax / 448, code = e4m3(x * (448 / amax))
 *   CGD_SCALE_POW2   scale = 2^k, the smallest power of two >= amax / 448,
 *                    code = e4m3(x * 2^-k)                      (round_scale)
 *   CGD_SCALE_UE8M0  as CGD_SCALE_POW2, the scale stored as the byte k + 127
 * with fp32 arithmetic throughout, correctly rounded division, the product
 * clamped to [-448, 448] and rounded to the nearest e4m3fn value (ties to
 * even). The cast back is bf16(code value * scale), the product in fp32.
 * Scale element (t, b) of an input lives at scales[t * scale_stride_token +
 * b * scale_stride_block] (row-major: H/128 and 1; column-major: 1 and T);
 * scales are fp32 (4 bytes) except UE8M0 (1 byte). Received scales are
 * row-major [recv_capacity, H/128]. All FP8 row pointers must be 16-byte
 * aligned; strides must be >= 0 and the caller guarantees every addressed
 * scale lies inside its buffer.
 * ------------------------------------------------------------------------- */

typedef enum { CGD_SCALE_F32 = 0, CGD_SCALE_POW2 = 1, CGD_SCALE_UE8M0 = 2 } cgd_scale_format;

/* per_token_cast_to_fp8: x bf16 [T, H] -> x_fp8 uint8 [T, H], x_scales. */
int cgd_cast_to_fp8(const void* x, int64_t num_tokens, int hidden, void* x_fp8, void* x_scales,
                    int64_t scale_stride_token, int64_t scale_stride_block, int scale_format, hipStream_t stream);

/* per_token_cast_back: (x_fp8, x_scales) -> out bf16 [T, H]. */
int cgd_cast_back(const void* x_fp8, const void* x_scales, int64_t scale_stride_token, int64_t scale_stride_block,
                  int scale_format, int64_t num_tokens, int hidden, void* out, hipStream_t stream);

/* Dispatch that casts on the way (the low-latency dispatch with FP8), to the
 * rows of a dst_row from cgd_dispatch_plan or an earlier dispatch: x is bf16
 * [T, H]; each chunk is cast once, exactly as cgd_cast_to_fp8 would, and its
 * codes and scales are written to every destination row: recv_x_fp8
 * [recv_capacity, H], recv_scales [recv_capacity, H/128]. */
int cgd_dispatch_cached_cast_fp8(const void* x, int64_t num_tokens, int hidden, int num_topk, int scale_format,
                                 const int32_t* dst_row, void* recv_x_fp8, void* recv_scales, int64_t recv_capacity,
                                 hipStream_t stream);

/* Non-cached dispatch that casts on the way (the dispatch of the "Dispatch
 * API" section of the Python interface notes with an FP8 payload, as the
 * low-latency dispatch with FP8 casts it): the plan of cgd_dispatch_plan
 * followed by the cast of cgd_dispatch_cached_cast_fp8 to the plan's rows, in
 * one call, so that the plan's idle compute units pull x into the caches
 * while it runs and the cast reads it from there. Arguments, outputs and
 * errors as cgd_dispatch, except: scale_format is 0 (fp32 amax/448), 1 (fp32
 * power of two) or 2 (UE8M0 byte); hidden must be a positive multiple of 128;
 * the rows go to recv_x_fp8 (uint8 e4m3fn codes [recv_capacity, hidden],
 * 16-byte aligned) and recv_scales ([recv_capacity, hidden/128], fp32 or one
 * byte for format 2), written for rows with data only; x is bf16 [num_tokens,
 * hidden]. The handle (expert_offset, recv_src_idx, dst_row) and
 * num_recv_tokens_per_expert are those of cgd_dispatch. */
int cgd_dispatch_cast_fp8(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx, int num_topk,
                          int num_experts, int num_ranks, int expert_alignment, int scale_format, void* recv_x_fp8,
                          void* recv_scales, int64_t recv_capacity, int32_t* expert_offset,
                          int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* dst_row,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* cgd_get_dispatch_layout and cgd_dispatch_cast_fp8 in one call: the layout
 * outputs (as cgd_get_dispatch_layout; no layout workspace is needed) come
 * from the plan's pass over the routing, as in cgd_layout_and_dispatch_plan;
 * everything else as cgd_dispatch_cast_fp8. */
int cgd_layout_and_dispatch_cast_fp8(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                     int num_topk, int num_experts, int num_ranks, int expert_alignment,
                                     int scale_format, void* recv_x_fp8, void* recv_scales, int64_t recv_capacity,
                                     int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                                     uint8_t* is_token_in_rank, int32_t* expert_offset,
                                     int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* dst_row,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Cached dispatch of the FP8 tuple with a dst_row from an earlier dispatch
 * or cgd_dispatch_plan: rows of H code bytes and the rows' scales move to
 * recv_x_fp8 [recv_capacity, H], recv_scales [recv_capacity, H/128]. */
int cgd_dispatch_cached_fp8(const void* x_fp8, const void* x_scales, int64_t scale_stride_token,
                            int64_t scale_stride_block, int scale_format, int64_t num_tokens, int hidden, int num_topk,
                            const int32_t* dst_row, void* recv_x_fp8, void* recv_scales, int64_t recv_capacity,
                            hipStream_t stream);

/* Normal-mode dispatch apply with the FP8 tuple as x (after
 * cgd_normal_dispatch_plan), and its cached form. */
int cgd_normal_dispatch_apply_fp8(const void* x_fp8, const void* x_scales, int64_t scale_stride_token,
                                  int64_t scale_stride_block, int scale_format, int64_t num_tokens, int hidden,
                                  const int64_t* topk_idx, const float* topk_weights, int num_topk, int num_experts,
                                  int num_ranks, void* recv_x_fp8, void* recv_scales, int64_t recv_capacity,
                                  const int32_t* rank_offset, int32_t* recv_src_idx, int32_t* send_row,
                                  int64_t* recv_topk_idx, float* recv_topk_weights, const void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

int cgd_normal_dispatch_cached_fp8(const void* x_fp8, const void* x_scales, int64_t scale_stride_token,
                                   int64_t scale_stride_block, int scale_format, int64_t num_tokens, int hidden,
                                   int num_ranks, const int32_t* send_row, void* recv_x_fp8, void* recv_scales,
                                   int64_t recv_capacity, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Fixed-capacity packed layout (the low-latency dispatch's receive buffers:
 * legacy test analysis page, low-latency dispatch call and per-expert check;
 * Python interface notes, "Dispatch API", num_worst_tokens).
 *
 * Expert e owns rows [e*expert_capacity, (e+1)*expert_capacity) of
 * packed_recv_x [num_experts, expert_capacity, hidden]; its valid rows come
 * first, in ascending (token, slot) order; a slot whose rank inside its expert
 * reaches expert_capacity is dropped (dst_row -1). Shapes depend only on the
 * sizes, so no host synchronisation is ever needed and a captured graph can
 * replay the call.
 *   packed_recv_count      int32 [num_experts] out: valid rows per expert
 *   recv_src_info          int32 [num_experts, expert_capacity] out: source token of each
 *                          valid row, -1 elsewhere (with one source the pages' layout range
 *                          per (expert, source) is (0, count) and is not produced)
 *   dst_row                int32 [num_tokens, num_topk] out: packed row of each slot, -1 if
 *                          not selected or dropped; cgd_combine with this dst_row and
 *                          recv_capacity = num_experts * expert_capacity combines packed
 *                          expert outputs (the low-latency combine)
 *   cumulative_recv_stats  int32 [num_experts] or NULL: packed_recv_count is added to it
 *                          (the pages' cumulative_local_expert_recv_stats)
 *   workspace              >= cgd_packed_workspace_bytes(...), same rules as the dispatch one
 * ------------------------------------------------------------------------- */
size_t cgd_packed_workspace_bytes(int64_t num_tokens, int num_topk, int num_experts);

int cgd_dispatch_packed(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx, int num_topk,
                        int num_experts, int num_ranks, int64_t expert_capacity, void* packed_recv_x,
                        int32_t* packed_recv_count, int32_t* recv_src_info, int32_t* dst_row,
                        int32_t* cumulative_recv_stats, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The packed layout with the FP8 cast on the way (the low-latency dispatch
 * with FP8): packed_recv_x_fp8 [num_experts * expert_capacity, hidden] codes,
 * packed_recv_scales [num_experts * expert_capacity, hidden/128]. */
int cgd_dispatch_packed_cast_fp8(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                 int num_topk, int num_experts, int num_ranks, int64_t expert_capacity,
                                 int scale_format, void* packed_recv_x_fp8, void* packed_recv_scales,
                                 int32_t* packed_recv_count, int32_t* recv_src_info, int32_t* dst_row,
                                 int32_t* cumulative_recv_stats, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* cgd_get_dispatch_layout and the packed dispatch in one call: the layout
 * outputs (as cgd_get_dispatch_layout; no layout workspace is needed) come
 * from the plan's pass over the routing, as in cgd_layout_and_dispatch (the
 * low-latency dispatch of the legacy tests, which follows the layout call of
 * the same routing); a batch of at most 256 tokens takes one launch.
 *   num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank
 *                           out, as cgd_get_dispatch_layout
 *   workspace               >= cgd_dispatch_workspace_bytes(num_tokens, num_topk,
 *                           num_experts, num_ranks), rules as the dispatch one
 * Everything else as cgd_dispatch_packed / cgd_dispatch_packed_cast_fp8. */
int cgd_layout_and_dispatch_packed(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                   int num_topk, int num_experts, int num_ranks, int64_t expert_capacity,
                                   void* packed_recv_x, int32_t* packed_recv_count, int32_t* recv_src_info,
                                   int32_t* dst_row, int32_t* cumulative_recv_stats, int32_t* num_tokens_per_rank,
                                   int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

int cgd_layout_and_dispatch_packed_cast_fp8(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                            int num_topk, int num_experts, int num_ranks, int64_t expert_capacity,
                                            int scale_format, void* packed_recv_x_fp8, void* packed_recv_scales,
                                            int32_t* packed_recv_count, int32_t* recv_src_info, int32_t* dst_row,
                                            int32_t* cumulative_recv_stats, int32_t* num_tokens_per_rank,
                                            int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* get_dispatch_layout and cgd_normal_dispatch_plan in one launch: the plan
 * needs only is_token_in_rank (and the per-expert counts for the aligned
 * receive counts), which the layout computes from the same tile of topk_idx
 * (Layout API "Return Values"; legacy tests, normal-mode dispatch call, whose
 * inputs are the layout outputs).
 *   outputs                 as cgd_get_dispatch_layout, and rank_offset [R+1]
 *                           and num_recv_tokens_per_expert [E] (may be NULL)
 *                           as cgd_normal_dispatch_plan
 *   workspace               >= cgd_layout_and_normal_workspace_bytes(...),
 *                           256-byte aligned; zero-fill and reuse rules as
 *                           the layout workspace;
 *                           it begins with the rank-granular plan's workspace:
 *                           pass the same pointer to cgd_normal_dispatch_apply
 *                           (or _apply_fp8), which reads the plan from it
 * Errors as cgd_get_dispatch_layout and cgd_normal_dispatch_plan. */
size_t cgd_layout_and_normal_workspace_bytes(int64_t num_tokens, int num_topk, int num_experts, int num_ranks);

int cgd_layout_and_normal_dispatch_plan(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                                        int num_ranks, int expert_alignment, int32_t* num_tokens_per_rank,
                                        int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                                        int32_t* rank_offset, int32_t* num_recv_tokens_per_expert, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/* cgd_layout_and_normal_dispatch_plan followed by cgd_normal_dispatch_apply
 * (the normal-mode dispatch of the legacy tests, whose inputs are the layout
 * outputs) in one call, so that the plan's idle compute units pull x into
 * the caches while it runs and the apply reads it from there. Arguments,
 * outputs and errors as those two calls (topk_idx feeds the layout; topk_weights,
 * recv_topk_idx and recv_topk_weights are all given or all NULL); the
 * workspace is that of cgd_layout_and_normal_dispatch_plan and afterwards
 * holds the plan, as there. A batch of at most 256 tokens takes one launch. */
int cgd_layout_and_normal_dispatch(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                   const float* topk_weights, int num_topk, int num_experts, int num_ranks,
                                   int expert_alignment, void* recv_x, int64_t recv_capacity,
                                   int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                                   uint8_t* is_token_in_rank, int32_t* rank_offset,
                                   int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* send_row,
                                   int64_t* recv_topk_idx, float* recv_topk_weights, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* cgd_layout_and_normal_dispatch with the FP8 payload cast on the way: the
 * plan's idle compute units cast x (bf16 [num_tokens, hidden]) per token, as
 * cgd_cast_to_fp8 would, into x_fp8 (e4m3fn codes [num_tokens, hidden],
 * 16-byte aligned) and x_scales (row-major [num_tokens, hidden/128], fp32, or
 * one byte for scale_format 2) while the plan runs, and the apply then moves
 * that tuple, as cgd_normal_dispatch_apply_fp8, to recv_x_fp8
 * [recv_capacity, hidden] and recv_scales [recv_capacity, hidden/128] (legacy
 * tests, normal-mode dispatch with the FP8 tuple as x; Python notes "Dispatch
 * API", the FP8 form of x). hidden must be a positive multiple of 128;
 * everything else as cgd_layout_and_normal_dispatch. */
int cgd_layout_and_normal_dispatch_cast_fp8(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                            const float* topk_weights, int num_topk, int num_experts, int num_ranks,
                                            int expert_alignment, int scale_format, void* x_fp8, void* x_scales,
                                            void* recv_x_fp8, void* recv_scales, int64_t recv_capacity,
                                            int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                                            uint8_t* is_token_in_rank, int32_t* rank_offset,
                                            int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx,
                                            int32_t* send_row, int64_t* recv_topk_idx, float* recv_topk_weights,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* -------------------------------------------------------------------------
 * cgd_copy: dst[0, bytes) = src[0, bytes), bitwise.
 * Not an operation of the method: a measured copy ceiling, reported beside
 * the spec peak that the dispatch and combine bandwidths are measured
 * against, with the data kernels' memory policy (16-byte non-temporal loads
 * and stores, one store per lane).
 *   src, dst  device pointers, 16-byte aligned, not overlapping; may be NULL
 *             when bytes == 0
 *   bytes     >= 0, a multiple of 16
 * Errors: CGD_ERR_INVALID_ARG (negative or unaligned size, misaligned or
 * null pointer), CGD_ERR_HIP (launch failure). Only enqueues on stream.
 * ------------------------------------------------------------------------- */
int cgd_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

/* -------------------------------------------------------------------------
 * cgd_empty: enqueues one kernel of one wave that does nothing.
 * Not an operation of the method: its launches measure the floor under the
 * latency-bound calls (get_dispatch_layout, the dispatch plan), timed the same
 * way as they are. Errors: CGD_ERR_HIP (launch failure). Only enqueues on
 * stream.
 * ------------------------------------------------------------------------- */
int cgd_empty(hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CGD_H */
