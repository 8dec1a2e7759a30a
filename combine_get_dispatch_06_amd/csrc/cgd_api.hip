// C-ABI entry points of libcgd: argument checks, workspace sizing, launches.
// Declarations and the contract of every call are in include/cgd.h.
#include "cgd.h"

#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "cgd_launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int hip_fail(hipError_t err, const char* what) {
    return fail(CGD_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Limits of the get_dispatch_layout API page ("Parameters", "Notes").
int check_routing_sizes(int64_t T, int K, int E, int R) {
    if (T < 0) return fail(CGD_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %lld)", (long long)T);
    if (K < 1 || K > cgd::kMaxTopk) return fail(CGD_ERR_INVALID_ARG, "num_topk must be in [1,16] (got %d)", K);
    if (E < 1 || E > cgd::kMaxExperts)
        return fail(CGD_ERR_INVALID_ARG, "num_experts must be in [1,512] (got %d)", E);
    if (R < 1 || R > cgd::kMaxRanks) return fail(CGD_ERR_INVALID_ARG, "num_ranks must be in [1,384] (got %d)", R);
    if (E % R != 0)
        return fail(CGD_ERR_INVALID_ARG, "num_experts (%d) must be divisible by num_ranks (%d)", E, R);
    if (T * (int64_t)K > INT32_MAX) return fail(CGD_ERR_INVALID_ARG, "num_tokens * num_topk exceeds INT32_MAX");
    return CGD_OK;
}

int check_hidden(int H) {
    if (H < 8 || H % 8 != 0) return fail(CGD_ERR_INVALID_ARG, "hidden must be a positive multiple of 8 (got %d)", H);
    return CGD_OK;
}

// A token reaches at most min(K, R) ranks.
int64_t normal_capacity_of(int64_t T, int K, int R) {
    if (T < 0 || K < 1 || R < 1) return -1;
    const int64_t cap = T * (int64_t)(K < R ? K : R);
    return cap > INT32_MAX ? -1 : cap;
}

int64_t capacity_of(int64_t T, int K, int E, int A) {
    if (T < 0 || K < 1 || E < 1 || A < 1) return -1;
    const int64_t cap = T * (int64_t)K + (int64_t)E * (int64_t)(A - 1);
    if (A > INT32_MAX / E || cap > INT32_MAX) return -1;
    return cap;
}

// FP8 payload: rows of H e4m3 bytes with H % 128 == 0, one scale per block
// of 128 channels (4-byte fp32, or 1-byte UE8M0 for format 2).
int check_fp8(int H, int fmt) {
    if (H < 128 || H % 128 != 0)
        return fail(CGD_ERR_INVALID_ARG, "FP8 payload needs hidden to be a positive multiple of 128 (got %d)", H);
    if (fmt < CGD_SCALE_F32 || fmt > CGD_SCALE_UE8M0)
        return fail(CGD_ERR_INVALID_ARG, "scale_format must be 0, 1 or 2 (got %d)", fmt);
    return CGD_OK;
}

int check_scales(const void* scales, int64_t st, int64_t sb, int fmt, bool needed) {
    if (needed && !scales) return fail(CGD_ERR_INVALID_ARG, "null scales");
    if (st < 0 || sb < 0) return fail(CGD_ERR_INVALID_ARG, "scale strides must be >= 0");
    if (!aligned(scales, fmt == CGD_SCALE_UE8M0 ? 1 : 4)) return fail(CGD_ERR_INVALID_ARG, "misaligned scales");
    return CGD_OK;
}

}  // namespace

extern "C" {

const char* cgd_version(void) { return "cgd 0.1.0 (gfx950)"; }

const char* cgd_last_error(void) { return g_last_error.c_str(); }

size_t cgd_layout_workspace_bytes(int64_t num_tokens, int num_topk, int num_experts, int num_ranks) {
    if (num_tokens < 0 || num_topk < 1 || num_experts < 1 || num_experts > cgd::kMaxExperts || num_ranks < 1 ||
        num_ranks > cgd::kMaxRanks)
        return 0;
    return cgd::layout_workspace_bytes(num_tokens, num_experts, num_ranks);
}

size_t cgd_dispatch_workspace_bytes(int64_t num_tokens, int num_topk, int num_experts, int num_ranks) {
    if (num_tokens < 0 || num_topk < 1 || num_experts < 1 || num_experts > cgd::kMaxExperts || num_ranks < 1 ||
        num_ranks > cgd::kMaxRanks)
        return 0;
    return cgd::dispatch_workspace_bytes(num_tokens, num_topk, num_experts, num_ranks);
}

int64_t cgd_dispatch_capacity(int64_t num_tokens, int num_topk, int num_experts, int expert_alignment) {
    return capacity_of(num_tokens, num_topk, num_experts, expert_alignment);
}

int cgd_get_dispatch_layout(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                            int num_ranks, int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                            uint8_t* is_token_in_rank, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    int rc = check_routing_sizes(num_tokens, num_topk, num_experts, num_ranks);
    if (rc) return rc;
    if (!num_tokens_per_rank || !num_tokens_per_expert)
        return fail(CGD_ERR_INVALID_ARG, "null count output pointer");
    if (num_tokens > 0 && (!topk_idx || !is_token_in_rank))
        return fail(CGD_ERR_INVALID_ARG, "null topk_idx or is_token_in_rank pointer");
    if (!aligned(topk_idx, 8) || !aligned(num_tokens_per_rank, 4) || !aligned(num_tokens_per_expert, 4))
        return fail(CGD_ERR_INVALID_ARG, "misaligned topk_idx or count output");
    if (!aligned(is_token_in_rank, 16)) return fail(CGD_ERR_INVALID_ARG, "is_token_in_rank must be 16-byte aligned");
    const size_t need = cgd::layout_workspace_bytes(num_tokens, num_experts, num_ranks);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(CGD_ERR_WORKSPACE, "layout workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                    workspace_bytes);
    hipError_t err = cgd::launch_layout(topk_idx, num_tokens, num_topk, num_experts, num_ranks, num_tokens_per_rank,
                                        num_tokens_per_expert, is_token_in_rank, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "layout launch");
    return CGD_OK;
}

// Checks shared by the dispatch entry points (all but the workspace).
static int check_plan_core(const int64_t* topk_idx, int64_t T, int K, int E, int R, int A, int64_t cap,
                           const int32_t* expert_offset, const int32_t* nrecv, const int32_t* recv_src_idx,
                           const int32_t* dst_row) {
    int rc = check_routing_sizes(T, K, E, R);
    if (rc) return rc;
    if (A < 1) return fail(CGD_ERR_INVALID_ARG, "expert_alignment must be >= 1");
    const int64_t need_rows = capacity_of(T, K, E, A);
    if (need_rows < 0) return fail(CGD_ERR_INVALID_ARG, "receive capacity for these sizes exceeds INT32_MAX");
    if (cap < need_rows || cap > INT32_MAX)
        return fail(CGD_ERR_CAPACITY, "recv_capacity must be in [%lld, INT32_MAX] (got %lld)", (long long)need_rows,
                    (long long)cap);
    if (!expert_offset) return fail(CGD_ERR_INVALID_ARG, "null expert_offset");
    if (T > 0 && (!topk_idx || !dst_row)) return fail(CGD_ERR_INVALID_ARG, "null topk_idx or dst_row");
    if (cap > 0 && !recv_src_idx) return fail(CGD_ERR_INVALID_ARG, "null recv_src_idx");
    if (!aligned(topk_idx, 8) || !aligned(expert_offset, 4) || !aligned(nrecv, 4) || !aligned(recv_src_idx, 4) ||
        !aligned(dst_row, 4))
        return fail(CGD_ERR_INVALID_ARG, "misaligned index pointer");
    return CGD_OK;
}

static int check_dispatch_workspace(int64_t T, int K, int E, int R, const void* workspace, size_t workspace_bytes) {
    const size_t need = cgd::dispatch_workspace_bytes(T, K, E, R);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(CGD_ERR_WORKSPACE, "dispatch workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                    workspace_bytes);
    return CGD_OK;
}

static int check_plan_args(const int64_t* topk_idx, int64_t T, int K, int E, int R, int A, int64_t cap,
                           const int32_t* expert_offset, const int32_t* nrecv, const int32_t* recv_src_idx,
                           const int32_t* dst_row, const void* workspace, size_t workspace_bytes) {
    int rc = check_plan_core(topk_idx, T, K, E, R, A, cap, expert_offset, nrecv, recv_src_idx, dst_row);
    if (rc) return rc;
    return check_dispatch_workspace(T, K, E, R, workspace, workspace_bytes);
}

// Checks of the row payload of a dispatch (x in, recv_x out).
static int check_rows_args(const void* x, int64_t T, int H, int64_t cap, const void* recv_x) {
    int rc = check_hidden(H);
    if (rc) return rc;
    if (T > 0 && !x) return fail(CGD_ERR_INVALID_ARG, "null x");
    if (cap > 0 && !recv_x) return fail(CGD_ERR_INVALID_ARG, "null recv_x");
    if (!aligned(x, 16) || !aligned(recv_x, 16)) return fail(CGD_ERR_INVALID_ARG, "x and recv_x must be 16-byte aligned");
    return CGD_OK;
}

int cgd_dispatch_plan(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts, int num_ranks,
                      int expert_alignment, int64_t recv_capacity, int32_t* expert_offset,
                      int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* dst_row, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    int rc = check_plan_args(topk_idx, num_tokens, num_topk, num_experts, num_ranks, expert_alignment, recv_capacity,
                             expert_offset, num_recv_tokens_per_expert, recv_src_idx, dst_row, workspace,
                             workspace_bytes);
    if (rc) return rc;
    hipError_t err = cgd::launch_dispatch_plan(topk_idx, num_tokens, num_topk, num_experts, expert_alignment,
                                               recv_capacity, expert_offset, num_recv_tokens_per_expert, recv_src_idx,
                                               dst_row, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "dispatch plan launch");
    return CGD_OK;
}

// Checks of get_dispatch_layout's outputs when another entry point produces them too.
static int check_layout_outputs(int64_t T, const int32_t* ntpr, const int32_t* ntpe, const uint8_t* itr) {
    if (!ntpr || !ntpe) return fail(CGD_ERR_INVALID_ARG, "null count output pointer");
    if (T > 0 && !itr) return fail(CGD_ERR_INVALID_ARG, "null is_token_in_rank");
    if (!aligned(ntpr, 4) || !aligned(ntpe, 4)) return fail(CGD_ERR_INVALID_ARG, "misaligned count output");
    if (!aligned(itr, 16)) return fail(CGD_ERR_INVALID_ARG, "is_token_in_rank must be 16-byte aligned");
    return CGD_OK;
}

int cgd_layout_and_dispatch_plan(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                                 int num_ranks, int expert_alignment, int64_t recv_capacity,
                                 int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                                 uint8_t* is_token_in_rank, int32_t* expert_offset,
                                 int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* dst_row,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = check_plan_args(topk_idx, num_tokens, num_topk, num_experts, num_ranks, expert_alignment, recv_capacity,
                             expert_offset, num_recv_tokens_per_expert, recv_src_idx, dst_row, workspace,
                             workspace_bytes);
    if (rc) return rc;
    if ((rc = check_layout_outputs(num_tokens, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank)))
        return rc;
    hipError_t err = cgd::launch_layout_and_plan(topk_idx, num_tokens, num_topk, num_experts, num_ranks,
                                                 expert_alignment, recv_capacity, num_tokens_per_rank,
                                                 num_tokens_per_expert, is_token_in_rank, expert_offset,
                                                 num_recv_tokens_per_expert, recv_src_idx, dst_row, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "layout and dispatch plan launch");
    return CGD_OK;
}

int cgd_dispatch(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx, int num_topk,
                 int num_experts, int num_ranks, int expert_alignment, void* recv_x, int64_t recv_capacity,
                 int32_t* expert_offset, int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* dst_row,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = check_plan_args(topk_idx, num_tokens, num_topk, num_experts, num_ranks, expert_alignment, recv_capacity,
                             expert_offset, num_recv_tokens_per_expert, recv_src_idx, dst_row, workspace,
                             workspace_bytes);
    if (rc) return rc;
    if ((rc = check_rows_args(x, num_tokens, hidden, recv_capacity, recv_x))) return rc;
    hipError_t err;
    if (cgd::dispatch_fuses(num_tokens)) {  // one tile: plan and apply in one launch
        err = cgd::launch_dispatch_fused(x, num_tokens, hidden, topk_idx, num_topk, num_experts, expert_alignment,
                                         recv_x, recv_capacity, expert_offset, num_recv_tokens_per_expert,
                                         recv_src_idx, dst_row, workspace, stream);
        if (err != hipSuccess) return hip_fail(err, "fused dispatch launch");
        return CGD_OK;
    }
    err = cgd::launch_dispatch_plan(topk_idx, num_tokens, num_topk, num_experts, expert_alignment, recv_capacity,
                                    expert_offset, num_recv_tokens_per_expert, recv_src_idx, dst_row, workspace,
                                    stream, x, num_tokens * (int64_t)hidden * 2);
    if (err != hipSuccess) return hip_fail(err, "dispatch plan launch");
    err = cgd::launch_dispatch_cached(x, num_tokens, hidden, num_topk, dst_row, recv_x, recv_capacity, stream, true);
    if (err != hipSuccess) return hip_fail(err, "dispatch row copy launch");
    return CGD_OK;
}

// Checks of cgd_layout_and_dispatch's arguments other than the workspace.
static int check_layout_and_dispatch(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E, int R,
                                     int A, const void* recv_x, int64_t cap, const int32_t* ntpr, const int32_t* ntpe,
                                     const uint8_t* itr, const int32_t* expert_offset, const int32_t* nrecv,
                                     const int32_t* recv_src_idx, const int32_t* dst_row) {
    int rc = check_plan_core(topk_idx, T, K, E, R, A, cap, expert_offset, nrecv, recv_src_idx, dst_row);
    if (rc) return rc;
    if ((rc = check_rows_args(x, T, H, cap, recv_x))) return rc;
    return check_layout_outputs(T, ntpr, ntpe, itr);
}

// cgd_layout_and_dispatch's launches, its arguments checked.
static int layout_and_dispatch_launches(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                        int num_topk, int num_experts, int num_ranks, int expert_alignment,
                                        void* recv_x, int64_t recv_capacity, int32_t* num_tokens_per_rank,
                                        int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                                        int32_t* expert_offset, int32_t* num_recv_tokens_per_expert,
                                        int32_t* recv_src_idx, int32_t* dst_row, void* workspace,
                                        hipStream_t stream) {
    hipError_t err;
    if (cgd::dispatch_fuses(num_tokens)) {  // one tile: layout, plan and rows in one launch
        err = cgd::launch_layout_and_dispatch_fused(x, num_tokens, hidden, topk_idx, num_topk, num_experts, num_ranks,
                                                    expert_alignment, recv_x, recv_capacity, num_tokens_per_rank,
                                                    num_tokens_per_expert, is_token_in_rank, expert_offset,
                                                    num_recv_tokens_per_expert, recv_src_idx, dst_row, workspace,
                                                    stream);
        if (err != hipSuccess) return hip_fail(err, "fused layout and dispatch launch");
        return CGD_OK;
    }
    err = cgd::launch_layout_and_plan(topk_idx, num_tokens, num_topk, num_experts, num_ranks, expert_alignment,
                                      recv_capacity, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank,
                                      expert_offset, num_recv_tokens_per_expert, recv_src_idx, dst_row, workspace,
                                      stream, x, num_tokens * (int64_t)hidden * 2);
    if (err != hipSuccess) return hip_fail(err, "layout and dispatch plan launch");
    err = cgd::launch_dispatch_cached(x, num_tokens, hidden, num_topk, dst_row, recv_x, recv_capacity, stream, true);
    if (err != hipSuccess) return hip_fail(err, "dispatch row copy launch");
    return CGD_OK;
}

int cgd_layout_and_dispatch(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx, int num_topk,
                            int num_experts, int num_ranks, int expert_alignment, void* recv_x,
                            int64_t recv_capacity, int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                            uint8_t* is_token_in_rank, int32_t* expert_offset, int32_t* num_recv_tokens_per_expert,
                            int32_t* recv_src_idx, int32_t* dst_row, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    int rc = check_layout_and_dispatch(x, num_tokens, hidden, topk_idx, num_topk, num_experts, num_ranks,
                                       expert_alignment, recv_x, recv_capacity, num_tokens_per_rank,
                                       num_tokens_per_expert, is_token_in_rank, expert_offset,
                                       num_recv_tokens_per_expert, recv_src_idx, dst_row);
    if (rc) return rc;
    if ((rc = check_dispatch_workspace(num_tokens, num_topk, num_experts, num_ranks, workspace, workspace_bytes)))
        return rc;
    return layout_and_dispatch_launches(x, num_tokens, hidden, topk_idx, num_topk, num_experts, num_ranks,
                                        expert_alignment, recv_x, recv_capacity, num_tokens_per_rank,
                                        num_tokens_per_expert, is_token_in_rank, expert_offset,
                                        num_recv_tokens_per_expert, recv_src_idx, dst_row, workspace, stream);
}

int cgd_dispatch_cached(const void* x, int64_t num_tokens, int hidden, int num_topk, const int32_t* dst_row,
                        void* recv_x, int64_t recv_capacity, hipStream_t stream) {
    if (num_tokens < 0) return fail(CGD_ERR_INVALID_ARG, "num_tokens must be >= 0");
    if (num_topk < 1 || num_topk > cgd::kMaxTopk) return fail(CGD_ERR_INVALID_ARG, "num_topk must be in [1,16]");
    int rc = check_hidden(hidden);
    if (rc) return rc;
    if (recv_capacity < 0 || recv_capacity > INT32_MAX)
        return fail(CGD_ERR_CAPACITY, "recv_capacity must be in [0, INT32_MAX]");
    if (num_tokens > 0 && (!x || !dst_row || (recv_capacity > 0 && !recv_x)))
        return fail(CGD_ERR_INVALID_ARG, "null pointer");
    if (!aligned(x, 16) || !aligned(recv_x, 16)) return fail(CGD_ERR_INVALID_ARG, "x and recv_x must be 16-byte aligned");
    if (!aligned(dst_row, 4)) return fail(CGD_ERR_INVALID_ARG, "misaligned dst_row");
    hipError_t err = cgd::launch_dispatch_cached(x, num_tokens, hidden, num_topk, dst_row, recv_x, recv_capacity,
                                                 stream);
    if (err != hipSuccess) return hip_fail(err, "cached dispatch launch");
    return CGD_OK;
}

int cgd_combine(const void* expert_out, int64_t recv_capacity, int hidden, const int32_t* dst_row,
                const float* topk_weights, int64_t num_tokens, int num_topk, void* combined_x,
                hipStream_t stream) {
    if (num_tokens < 0) return fail(CGD_ERR_INVALID_ARG, "num_tokens must be >= 0");
    if (num_topk < 1 || num_topk > cgd::kMaxTopk) return fail(CGD_ERR_INVALID_ARG, "num_topk must be in [1,16]");
    int rc = check_hidden(hidden);
    if (rc) return rc;
    if (recv_capacity < 0 || recv_capacity > INT32_MAX)
        return fail(CGD_ERR_CAPACITY, "recv_capacity must be in [0, INT32_MAX]");
    if (num_tokens > 0 && (!dst_row || !topk_weights || !combined_x || (recv_capacity > 0 && !expert_out)))
        return fail(CGD_ERR_INVALID_ARG, "null pointer");
    if (!aligned(expert_out, 16) || !aligned(combined_x, 16))
        return fail(CGD_ERR_INVALID_ARG, "expert_out and combined_x must be 16-byte aligned");
    if (!aligned(dst_row, 4) || !aligned(topk_weights, 4)) return fail(CGD_ERR_INVALID_ARG, "misaligned index pointer");
    hipError_t err = cgd::launch_combine(expert_out, recv_capacity, hidden, dst_row, topk_weights, num_tokens,
                                         num_topk, combined_x, stream);
    if (err != hipSuccess) return hip_fail(err, "combine launch");
    return CGD_OK;
}

size_t cgd_normal_workspace_bytes(int64_t num_tokens, int num_ranks) {
    if (num_tokens < 0 || num_ranks < 1 || num_ranks > cgd::kMaxRanks) return 0;
    return cgd::normal_workspace_bytes(num_tokens, num_ranks);
}

int64_t cgd_normal_capacity(int64_t num_tokens, int num_topk, int num_ranks) {
    return normal_capacity_of(num_tokens, num_topk, num_ranks);
}

// Checks of the normal-mode plan (routing-independent sizes and the layout inputs).
static int check_normal_plan_args(const uint8_t* itr, int64_t T, int R, const int32_t* ntpe, int E, int A,
                                  const int32_t* rank_offset, const int32_t* nrecv, const void* workspace,
                                  size_t workspace_bytes) {
    if (T < 0) return fail(CGD_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %lld)", (long long)T);
    if (E < 1 || E > cgd::kMaxExperts)
        return fail(CGD_ERR_INVALID_ARG, "num_experts must be in [1,512] (got %d)", E);
    if (R < 1 || R > cgd::kMaxRanks) return fail(CGD_ERR_INVALID_ARG, "num_ranks must be in [1,384] (got %d)", R);
    if (E % R != 0)
        return fail(CGD_ERR_INVALID_ARG, "num_experts (%d) must be divisible by num_ranks (%d)", E, R);
    if (A < 1) return fail(CGD_ERR_INVALID_ARG, "expert_alignment must be >= 1");
    if (!rank_offset) return fail(CGD_ERR_INVALID_ARG, "null rank_offset");
    if (T > 0 && !itr) return fail(CGD_ERR_INVALID_ARG, "null is_token_in_rank");
    if ((ntpe == nullptr) != (nrecv == nullptr))
        return fail(CGD_ERR_INVALID_ARG, "num_tokens_per_expert and num_recv_tokens_per_expert go together");
    if (!aligned(rank_offset, 4) || !aligned(ntpe, 4) || !aligned(nrecv, 4))
        return fail(CGD_ERR_INVALID_ARG, "misaligned count pointer");
    const size_t need = cgd::normal_workspace_bytes(T, R);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(CGD_ERR_WORKSPACE, "normal dispatch workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                    workspace_bytes);
    return CGD_OK;
}

size_t cgd_layout_and_normal_workspace_bytes(int64_t num_tokens, int num_topk, int num_experts, int num_ranks) {
    if (cgd_layout_workspace_bytes(num_tokens, num_topk, num_experts, num_ranks) == 0) return 0;  // invalid sizes
    return cgd::normal_workspace_bytes(num_tokens, num_ranks) +
           cgd::layout_partial_bytes(num_tokens, num_experts, num_ranks);
}

// Checks of the layout + rank-granular plan's routing, layout outputs, rank
// offsets and workspace.
static int check_layout_and_normal_plan_args(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                                             int num_experts, int num_ranks, int expert_alignment,
                                             const int32_t* num_tokens_per_rank, const int32_t* num_tokens_per_expert,
                                             const uint8_t* is_token_in_rank, const int32_t* rank_offset,
                                             const int32_t* num_recv_tokens_per_expert, const void* workspace,
                                             size_t workspace_bytes) {
    int rc = check_routing_sizes(num_tokens, num_topk, num_experts, num_ranks);
    if (rc) return rc;
    if (expert_alignment < 1) return fail(CGD_ERR_INVALID_ARG, "expert_alignment must be >= 1");
    if (!num_tokens_per_rank || !num_tokens_per_expert || !rank_offset)
        return fail(CGD_ERR_INVALID_ARG, "null count or rank_offset pointer");
    if (num_tokens > 0 && (!topk_idx || !is_token_in_rank))
        return fail(CGD_ERR_INVALID_ARG, "null topk_idx or is_token_in_rank pointer");
    if (!aligned(topk_idx, 8) || !aligned(num_tokens_per_rank, 4) || !aligned(num_tokens_per_expert, 4) ||
        !aligned(rank_offset, 4) || !aligned(num_recv_tokens_per_expert, 4))
        return fail(CGD_ERR_INVALID_ARG, "misaligned topk_idx or count output");
    if (!aligned(is_token_in_rank, 16)) return fail(CGD_ERR_INVALID_ARG, "is_token_in_rank must be 16-byte aligned");
    const size_t need = cgd_layout_and_normal_workspace_bytes(num_tokens, num_topk, num_experts, num_ranks);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(CGD_ERR_WORKSPACE, "layout + normal plan workspace needs %zu bytes, 256-byte aligned (got %zu)",
                    need, workspace_bytes);
    return CGD_OK;
}

int cgd_layout_and_normal_dispatch_plan(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                                        int num_ranks, int expert_alignment, int32_t* num_tokens_per_rank,
                                        int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                                        int32_t* rank_offset, int32_t* num_recv_tokens_per_expert, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
    int rc = check_layout_and_normal_plan_args(topk_idx, num_tokens, num_topk, num_experts, num_ranks,
                                               expert_alignment, num_tokens_per_rank, num_tokens_per_expert,
                                               is_token_in_rank, rank_offset, num_recv_tokens_per_expert, workspace,
                                               workspace_bytes);
    if (rc) return rc;
    hipError_t err = cgd::launch_layout_and_normal_plan(topk_idx, num_tokens, num_topk, num_experts, num_ranks,
                                                        expert_alignment, num_tokens_per_rank, num_tokens_per_expert,
                                                        is_token_in_rank, rank_offset, num_recv_tokens_per_expert,
                                                        workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "layout and normal dispatch plan launch");
    return CGD_OK;
}

// Checks of the normal-mode apply (rows and per-row outputs).
static int check_normal_apply_args(const void* x, int64_t T, int H, const int64_t* topk_idx, const float* topk_w,
                                   int K, int E, int R, const void* recv_x, int64_t cap, const int32_t* rank_offset,
                                   const int32_t* recv_src_idx, const int32_t* send_row, const int64_t* recv_topk_idx,
                                   const float* recv_topk_w, const void* workspace, size_t workspace_bytes) {
    int rc = check_routing_sizes(T, K, E, R);
    if (rc) return rc;
    if ((rc = check_hidden(H))) return rc;
    const int64_t need_rows = normal_capacity_of(T, K, R);
    if (need_rows < 0) return fail(CGD_ERR_INVALID_ARG, "receive capacity for these sizes exceeds INT32_MAX");
    if (cap < need_rows || cap > INT32_MAX)
        return fail(CGD_ERR_CAPACITY, "recv_capacity must be in [%lld, INT32_MAX] (got %lld)", (long long)need_rows,
                    (long long)cap);
    if (!rank_offset) return fail(CGD_ERR_INVALID_ARG, "null rank_offset");
    if (T > 0 && (!x || !send_row)) return fail(CGD_ERR_INVALID_ARG, "null x or send_row");
    if (cap > 0 && (!recv_x || !recv_src_idx)) return fail(CGD_ERR_INVALID_ARG, "null receive pointer");
    // with top-k: recv_topk_* are given (both), and so are topk_* unless
    // there are no tokens (an empty tensor may have a null data pointer)
    const bool with_topk = recv_topk_idx != nullptr || recv_topk_w != nullptr;
    if (with_topk && (!recv_topk_idx || !recv_topk_w))
        return fail(CGD_ERR_INVALID_ARG, "recv_topk_idx and recv_topk_weights go together");
    if (T > 0 && ((topk_idx != nullptr) != with_topk || (topk_w != nullptr) != with_topk))
        return fail(CGD_ERR_INVALID_ARG,
                    "topk_idx, topk_weights, recv_topk_idx and recv_topk_weights must be all given or all null");
    if (!with_topk && (topk_idx || topk_w))
        return fail(CGD_ERR_INVALID_ARG, "topk_idx given without recv_topk_idx / recv_topk_weights");
    if (!aligned(x, 16) || !aligned(recv_x, 16)) return fail(CGD_ERR_INVALID_ARG, "x and recv_x must be 16-byte aligned");
    if (!aligned(topk_idx, 8) || !aligned(recv_topk_idx, 8) || !aligned(topk_w, 4) || !aligned(recv_topk_w, 4) ||
        !aligned(rank_offset, 4) || !aligned(recv_src_idx, 4) || !aligned(send_row, 4))
        return fail(CGD_ERR_INVALID_ARG, "misaligned index or weight pointer");
    const size_t need = cgd::normal_workspace_bytes(T, R);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(CGD_ERR_WORKSPACE, "normal dispatch workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                    workspace_bytes);
    return CGD_OK;
}

int cgd_normal_dispatch_plan(const uint8_t* is_token_in_rank, int64_t num_tokens, int num_ranks,
                             const int32_t* num_tokens_per_expert, int num_experts, int expert_alignment,
                             int32_t* rank_offset, int32_t* num_recv_tokens_per_expert, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    int rc = check_normal_plan_args(is_token_in_rank, num_tokens, num_ranks, num_tokens_per_expert, num_experts,
                                    expert_alignment, rank_offset, num_recv_tokens_per_expert, workspace,
                                    workspace_bytes);
    if (rc) return rc;
    hipError_t err = cgd::launch_normal_plan(is_token_in_rank, num_tokens, num_ranks, num_tokens_per_expert,
                                             num_experts, expert_alignment, rank_offset, num_recv_tokens_per_expert,
                                             workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "normal dispatch plan launch");
    return CGD_OK;
}

int cgd_normal_dispatch_apply(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                              const float* topk_weights, int num_topk, int num_experts, int num_ranks, void* recv_x,
                              int64_t recv_capacity, const int32_t* rank_offset, int32_t* recv_src_idx,
                              int32_t* send_row, int64_t* recv_topk_idx, float* recv_topk_weights,
                              const void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = check_normal_apply_args(x, num_tokens, hidden, topk_idx, topk_weights, num_topk, num_experts, num_ranks,
                                     recv_x, recv_capacity, rank_offset, recv_src_idx, send_row, recv_topk_idx,
                                     recv_topk_weights, workspace, workspace_bytes);
    if (rc) return rc;
    hipError_t err = cgd::launch_normal_apply(x, num_tokens, hidden, topk_idx, topk_weights, num_topk, num_experts,
                                              num_ranks, recv_x, recv_capacity, rank_offset, recv_src_idx, send_row,
                                              recv_topk_idx, recv_topk_weights, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "normal dispatch apply launch");
    return CGD_OK;
}

int cgd_layout_and_normal_dispatch(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                   const float* topk_weights, int num_topk, int num_experts, int num_ranks,
                                   int expert_alignment, void* recv_x, int64_t recv_capacity,
                                   int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                                   uint8_t* is_token_in_rank, int32_t* rank_offset,
                                   int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* send_row,
                                   int64_t* recv_topk_idx, float* recv_topk_weights, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    int rc = check_layout_and_normal_plan_args(topk_idx, num_tokens, num_topk, num_experts, num_ranks,
                                               expert_alignment, num_tokens_per_rank, num_tokens_per_expert,
                                               is_token_in_rank, rank_offset, num_recv_tokens_per_expert, workspace,
                                               workspace_bytes);
    if (rc) return rc;
    if ((rc = check_normal_apply_args(x, num_tokens, hidden, recv_topk_idx ? topk_idx : nullptr, topk_weights,
                                      num_topk, num_experts, num_ranks, recv_x, recv_capacity, rank_offset,
                                      recv_src_idx, send_row, recv_topk_idx, recv_topk_weights, workspace,
                                      workspace_bytes)))
        return rc;
    if (cgd::normal_dispatch_fuses(num_tokens)) {  // one tile (decode): layout, plan and rows in one launch
        const hipError_t err = cgd::launch_layout_and_normal_fused(
            x, num_tokens, hidden, topk_idx, recv_topk_idx ? topk_weights : nullptr, num_topk, num_experts, num_ranks,
            expert_alignment, recv_x, recv_capacity, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank,
            rank_offset, num_recv_tokens_per_expert, recv_src_idx, send_row, recv_topk_idx, recv_topk_weights,
            workspace, stream);
        return err == hipSuccess ? CGD_OK : hip_fail(err, "layout and normal dispatch launch");
    }
    hipError_t err = cgd::launch_layout_and_normal_plan(topk_idx, num_tokens, num_topk, num_experts, num_ranks,
                                                        expert_alignment, num_tokens_per_rank, num_tokens_per_expert,
                                                        is_token_in_rank, rank_offset, num_recv_tokens_per_expert,
                                                        workspace, stream, x, num_tokens * (int64_t)hidden * 2);
    if (err != hipSuccess) return hip_fail(err, "layout and normal dispatch plan launch");
    err = cgd::launch_normal_apply(x, num_tokens, hidden, recv_topk_idx ? topk_idx : nullptr, topk_weights, num_topk,
                                   num_experts, num_ranks, recv_x, recv_capacity, rank_offset, recv_src_idx, send_row,
                                   recv_topk_idx, recv_topk_weights, workspace, stream,
                                   cgd::normal_plan_prefetches(num_tokens, num_tokens * (int64_t)hidden * 2));
    if (err != hipSuccess) return hip_fail(err, "normal dispatch apply launch");
    return CGD_OK;
}

int cgd_layout_and_normal_dispatch_cast_fp8(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                            const float* topk_weights, int num_topk, int num_experts, int num_ranks,
                                            int expert_alignment, int scale_format, void* x_fp8, void* x_scales,
                                            void* recv_x_fp8, void* recv_scales, int64_t recv_capacity,
                                            int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                                            uint8_t* is_token_in_rank, int32_t* rank_offset,
                                            int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx,
                                            int32_t* send_row, int64_t* recv_topk_idx, float* recv_topk_weights,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = check_layout_and_normal_plan_args(topk_idx, num_tokens, num_topk, num_experts, num_ranks,
                                               expert_alignment, num_tokens_per_rank, num_tokens_per_expert,
                                               is_token_in_rank, rank_offset, num_recv_tokens_per_expert, workspace,
                                               workspace_bytes);
    if (rc) return rc;
    if ((rc = check_fp8(hidden, scale_format))) return rc;
    if (num_tokens > 0 && (!x || !x_fp8)) return fail(CGD_ERR_INVALID_ARG, "null x or x_fp8");
    if (!aligned(x, 16) || !aligned(x_fp8, 16)) return fail(CGD_ERR_INVALID_ARG, "x and x_fp8 must be 16-byte aligned");
    if ((rc = check_scales(x_scales, 0, 0, scale_format, num_tokens > 0))) return rc;
    // the apply reads the cast tuple (codes, row-major scales) and writes the FP8 rows
    if ((rc = check_normal_apply_args(x_fp8, num_tokens, hidden, recv_topk_idx ? topk_idx : nullptr,
                                      topk_weights, num_topk, num_experts, num_ranks, recv_x_fp8, recv_capacity,
                                      rank_offset, recv_src_idx, send_row, recv_topk_idx, recv_topk_weights,
                                      workspace, workspace_bytes)))
        return rc;
    if ((rc = check_scales(recv_scales, 0, 0, scale_format, num_tokens > 0 && recv_capacity > 0))) return rc;
    const cgd::NormalCast cast{x, hidden, scale_format, x_fp8, x_scales};
    if (cgd::normal_dispatch_fuses(num_tokens)) {  // one tile (decode): layout, plan, cast and rows in one launch
        const hipError_t err = cgd::launch_layout_and_normal_fused(
            x, num_tokens, hidden, topk_idx, recv_topk_idx ? topk_weights : nullptr, num_topk, num_experts, num_ranks,
            expert_alignment, recv_x_fp8, recv_capacity, num_tokens_per_rank, num_tokens_per_expert,
            is_token_in_rank, rank_offset, num_recv_tokens_per_expert, recv_src_idx, send_row, recv_topk_idx,
            recv_topk_weights, workspace, stream, &cast, recv_scales);
        return err == hipSuccess ? CGD_OK : hip_fail(err, "layout, normal dispatch and cast launch");
    }
    hipError_t err = cgd::launch_layout_and_normal_plan(topk_idx, num_tokens, num_topk, num_experts, num_ranks,
                                                        expert_alignment, num_tokens_per_rank, num_tokens_per_expert,
                                                        is_token_in_rank, rank_offset, num_recv_tokens_per_expert,
                                                        workspace, stream, nullptr, 0, &cast);
    if (err != hipSuccess) return hip_fail(err, "layout, normal dispatch plan and cast launch");
    if (num_tokens > 0 && !cgd::normal_plan_casts(num_tokens)) {  // a one-tile plan: the cast on its own
        err = cgd::launch_cast_to_fp8(x, num_tokens, hidden, x_fp8, x_scales, hidden / 128, 1, scale_format, stream);
        if (err != hipSuccess) return hip_fail(err, "cast launch");
    }
    err = cgd::launch_normal_apply_fp8(x_fp8, x_scales, hidden / 128, 1, scale_format, num_tokens, hidden,
                                       recv_topk_idx ? topk_idx : nullptr, topk_weights, num_topk, num_experts,
                                       num_ranks, recv_x_fp8, recv_scales, recv_capacity, rank_offset, recv_src_idx,
                                       send_row, recv_topk_idx, recv_topk_weights, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "normal FP8 dispatch apply launch");
    return CGD_OK;
}

int cgd_normal_dispatch(const void* x, int64_t num_tokens, int hidden, const uint8_t* is_token_in_rank,
                        const int32_t* num_tokens_per_expert, const int64_t* topk_idx, const float* topk_weights,
                        int num_topk, int num_experts, int num_ranks, int expert_alignment, void* recv_x,
                        int64_t recv_capacity, int32_t* rank_offset, int32_t* recv_src_idx, int32_t* send_row,
                        int64_t* recv_topk_idx, float* recv_topk_weights, int32_t* num_recv_tokens_per_expert,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = check_normal_plan_args(is_token_in_rank, num_tokens, num_ranks, num_tokens_per_expert, num_experts,
                                    expert_alignment, rank_offset, num_recv_tokens_per_expert, workspace,
                                    workspace_bytes);
    if (rc) return rc;
    if ((rc = check_normal_apply_args(x, num_tokens, hidden, topk_idx, topk_weights, num_topk, num_experts, num_ranks,
                                      recv_x, recv_capacity, rank_offset, recv_src_idx, send_row, recv_topk_idx,
                                      recv_topk_weights, workspace, workspace_bytes)))
        return rc;
    hipError_t err = cgd::launch_normal_plan(is_token_in_rank, num_tokens, num_ranks, num_tokens_per_expert,
                                             num_experts, expert_alignment, rank_offset, num_recv_tokens_per_expert,
                                             workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "normal dispatch plan launch");
    err = cgd::launch_normal_apply(x, num_tokens, hidden, topk_idx, topk_weights, num_topk, num_experts, num_ranks,
                                   recv_x, recv_capacity, rank_offset, recv_src_idx, send_row, recv_topk_idx,
                                   recv_topk_weights, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "normal dispatch apply launch");
    return CGD_OK;
}

int cgd_normal_dispatch_cached(const void* x, int64_t num_tokens, int hidden, int num_ranks, const int32_t* send_row,
                               void* recv_x, int64_t recv_capacity, hipStream_t stream) {
    if (num_tokens < 0) return fail(CGD_ERR_INVALID_ARG, "num_tokens must be >= 0");
    if (num_ranks < 1 || num_ranks > cgd::kMaxRanks) return fail(CGD_ERR_INVALID_ARG, "num_ranks must be in [1,384]");
    int rc = check_hidden(hidden);
    if (rc) return rc;
    if (recv_capacity < 0 || recv_capacity > INT32_MAX)
        return fail(CGD_ERR_CAPACITY, "recv_capacity must be in [0, INT32_MAX]");
    if (num_tokens > 0 && (!x || !send_row || (recv_capacity > 0 && !recv_x)))
        return fail(CGD_ERR_INVALID_ARG, "null pointer");
    if (!aligned(x, 16) || !aligned(recv_x, 16)) return fail(CGD_ERR_INVALID_ARG, "x and recv_x must be 16-byte aligned");
    if (!aligned(send_row, 4)) return fail(CGD_ERR_INVALID_ARG, "misaligned send_row");
    hipError_t err = cgd::launch_normal_dispatch_cached(x, num_tokens, hidden, num_ranks, send_row, recv_x,
                                                        recv_capacity, stream);
    if (err != hipSuccess) return hip_fail(err, "cached normal dispatch launch");
    return CGD_OK;
}

int cgd_normal_combine(const void* expert_out, int64_t recv_rows, int hidden, const int32_t* send_row,
                       int64_t num_tokens, int num_ranks, const float* recv_topk_weights, int num_topk,
                       const void* bias_0, const void* bias_1, void* combined_x, float* combined_topk_weights,
                       hipStream_t stream) {
    if (num_tokens < 0) return fail(CGD_ERR_INVALID_ARG, "num_tokens must be >= 0");
    if (num_ranks < 1 || num_ranks > cgd::kMaxRanks) return fail(CGD_ERR_INVALID_ARG, "num_ranks must be in [1,384]");
    if (num_topk < 1 || num_topk > cgd::kMaxTopk) return fail(CGD_ERR_INVALID_ARG, "num_topk must be in [1,16]");
    int rc = check_hidden(hidden);
    if (rc) return rc;
    if (recv_rows < 0 || recv_rows > INT32_MAX) return fail(CGD_ERR_CAPACITY, "recv_rows must be in [0, INT32_MAX]");
    // the weight pair goes together; an empty tensor may have a null pointer
    if (num_tokens > 0 && recv_topk_weights && !combined_topk_weights)
        return fail(CGD_ERR_INVALID_ARG, "recv_topk_weights given without combined_topk_weights");
    if (num_tokens > 0 && recv_rows > 0 && combined_topk_weights && !recv_topk_weights)
        return fail(CGD_ERR_INVALID_ARG, "combined_topk_weights requested without recv_topk_weights");
    if (num_tokens > 0 && (!send_row || !combined_x || (recv_rows > 0 && !expert_out)))
        return fail(CGD_ERR_INVALID_ARG, "null pointer");
    if (!aligned(expert_out, 16) || !aligned(combined_x, 16) || !aligned(bias_0, 16) || !aligned(bias_1, 16))
        return fail(CGD_ERR_INVALID_ARG, "expert_out, bias and combined_x must be 16-byte aligned");
    if (!aligned(send_row, 4) || !aligned(recv_topk_weights, 4) || !aligned(combined_topk_weights, 4))
        return fail(CGD_ERR_INVALID_ARG, "misaligned index or weight pointer");
    hipError_t err = cgd::launch_normal_combine(expert_out, recv_rows, hidden, send_row, num_tokens, num_ranks,
                                                recv_topk_weights, num_topk, bias_0, bias_1, combined_x,
                                                combined_topk_weights, stream);
    if (err != hipSuccess) return hip_fail(err, "normal combine launch");
    return CGD_OK;
}

int cgd_cast_to_fp8(const void* x, int64_t num_tokens, int hidden, void* x_fp8, void* x_scales,
                    int64_t scale_stride_token, int64_t scale_stride_block, int scale_format, hipStream_t stream) {
    if (num_tokens < 0) return fail(CGD_ERR_INVALID_ARG, "num_tokens must be >= 0");
    int rc = check_fp8(hidden, scale_format);
    if (rc) return rc;
    if ((rc = check_scales(x_scales, scale_stride_token, scale_stride_block, scale_format, num_tokens > 0))) return rc;
    if (num_tokens > 0 && (!x || !x_fp8)) return fail(CGD_ERR_INVALID_ARG, "null x or x_fp8");
    if (!aligned(x, 16) || !aligned(x_fp8, 16)) return fail(CGD_ERR_INVALID_ARG, "x and x_fp8 must be 16-byte aligned");
    hipError_t err = cgd::launch_cast_to_fp8(x, num_tokens, hidden, x_fp8, x_scales, scale_stride_token,
                                             scale_stride_block, scale_format, stream);
    if (err != hipSuccess) return hip_fail(err, "cast launch");
    return CGD_OK;
}

int cgd_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    if (bytes < 0 || bytes % 16 != 0) return fail(CGD_ERR_INVALID_ARG, "bytes must be a non-negative multiple of 16");
    if (bytes == 0) return CGD_OK;
    if (!src || !dst) return fail(CGD_ERR_INVALID_ARG, "null src or dst");
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(CGD_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
    hipError_t err = cgd::launch_copy(src, dst, bytes, stream);
    if (err != hipSuccess) return hip_fail(err, "copy launch");
    return CGD_OK;
}

int cgd_empty(hipStream_t stream) {
    hipError_t err = cgd::launch_empty(stream);
    if (err != hipSuccess) return hip_fail(err, "empty kernel launch");
    return CGD_OK;
}

int cgd_cast_back(const void* x_fp8, const void* x_scales, int64_t scale_stride_token, int64_t scale_stride_block,
                  int scale_format, int64_t num_tokens, int hidden, void* out, hipStream_t stream) {
    if (num_tokens < 0) return fail(CGD_ERR_INVALID_ARG, "num_tokens must be >= 0");
    int rc = check_fp8(hidden, scale_format);
    if (rc) return rc;
    if ((rc = check_scales(x_scales, scale_stride_token, scale_stride_block, scale_format, num_tokens > 0))) return rc;
    if (num_tokens > 0 && (!x_fp8 || !out)) return fail(CGD_ERR_INVALID_ARG, "null x_fp8 or out");
    if (!aligned(x_fp8, 16) || !aligned(out, 16)) return fail(CGD_ERR_INVALID_ARG, "x_fp8 and out must be 16-byte aligned");
    hipError_t err = cgd::launch_cast_back(x_fp8, x_scales, scale_stride_token, scale_stride_block, scale_format,
                                           num_tokens, hidden, out, stream);
    if (err != hipSuccess) return hip_fail(err, "cast back launch");
    return CGD_OK;
}

int cgd_dispatch_cached_cast_fp8(const void* x, int64_t num_tokens, int hidden, int num_topk, int scale_format,
                                 const int32_t* dst_row, void* recv_x_fp8, void* recv_scales, int64_t recv_capacity,
                                 hipStream_t stream) {
    if (num_tokens < 0) return fail(CGD_ERR_INVALID_ARG, "num_tokens must be >= 0");
    if (num_topk < 1 || num_topk > cgd::kMaxTopk) return fail(CGD_ERR_INVALID_ARG, "num_topk must be in [1,16]");
    int rc = check_fp8(hidden, scale_format);
    if (rc) return rc;
    if (recv_capacity < 0 || recv_capacity > INT32_MAX)
        return fail(CGD_ERR_CAPACITY, "recv_capacity must be in [0, INT32_MAX]");
    if (num_tokens > 0 && (!x || !dst_row || (recv_capacity > 0 && !recv_x_fp8)))
        return fail(CGD_ERR_INVALID_ARG, "null pointer");
    if (!aligned(x, 16) || !aligned(recv_x_fp8, 16))
        return fail(CGD_ERR_INVALID_ARG, "x and recv_x_fp8 must be 16-byte aligned");
    if (!aligned(dst_row, 4)) return fail(CGD_ERR_INVALID_ARG, "misaligned dst_row");
    if ((rc = check_scales(recv_scales, 0, 0, scale_format, num_tokens > 0 && recv_capacity > 0))) return rc;
    hipError_t err = cgd::launch_dispatch_cached_cast_fp8(x, num_tokens, hidden, num_topk, scale_format, dst_row,
                                                          recv_x_fp8, recv_scales, recv_capacity, stream);
    if (err != hipSuccess) return hip_fail(err, "FP8 cast dispatch launch");
    return CGD_OK;
}

// Checks of a cast-on-dispatch payload: bf16 x in, FP8 rows and scales out.
static int check_cast_rows(const void* x, int64_t T, int H, int fmt, int64_t cap, const void* recv_q,
                           const void* recv_s) {
    int rc = check_fp8(H, fmt);
    if (rc) return rc;
    if (T > 0 && !x) return fail(CGD_ERR_INVALID_ARG, "null x");
    if (cap > 0 && !recv_q) return fail(CGD_ERR_INVALID_ARG, "null recv_x_fp8");
    if (!aligned(x, 16) || !aligned(recv_q, 16))
        return fail(CGD_ERR_INVALID_ARG, "x and recv_x_fp8 must be 16-byte aligned");
    return check_scales(recv_s, 0, 0, fmt, T > 0 && cap > 0);
}

int cgd_dispatch_cast_fp8(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx, int num_topk,
                          int num_experts, int num_ranks, int expert_alignment, int scale_format, void* recv_x_fp8,
                          void* recv_scales, int64_t recv_capacity, int32_t* expert_offset,
                          int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* dst_row,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = check_plan_args(topk_idx, num_tokens, num_topk, num_experts, num_ranks, expert_alignment, recv_capacity,
                             expert_offset, num_recv_tokens_per_expert, recv_src_idx, dst_row, workspace,
                             workspace_bytes);
    if (rc) return rc;
    if ((rc = check_cast_rows(x, num_tokens, hidden, scale_format, recv_capacity, recv_x_fp8, recv_scales))) return rc;
    hipError_t err = cgd::launch_dispatch_cast_fp8(x, num_tokens, hidden, topk_idx, num_topk, num_experts,
                                                   expert_alignment, scale_format, recv_x_fp8, recv_scales,
                                                   recv_capacity, expert_offset, num_recv_tokens_per_expert,
                                                   recv_src_idx, dst_row, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "FP8 cast dispatch launch");
    return CGD_OK;
}

int cgd_layout_and_dispatch_cast_fp8(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                     int num_topk, int num_experts, int num_ranks, int expert_alignment,
                                     int scale_format, void* recv_x_fp8, void* recv_scales, int64_t recv_capacity,
                                     int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                                     uint8_t* is_token_in_rank, int32_t* expert_offset,
                                     int32_t* num_recv_tokens_per_expert, int32_t* recv_src_idx, int32_t* dst_row,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = check_plan_args(topk_idx, num_tokens, num_topk, num_experts, num_ranks, expert_alignment, recv_capacity,
                             expert_offset, num_recv_tokens_per_expert, recv_src_idx, dst_row, workspace,
                             workspace_bytes);
    if (rc) return rc;
    if ((rc = check_layout_outputs(num_tokens, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank)))
        return rc;
    if ((rc = check_cast_rows(x, num_tokens, hidden, scale_format, recv_capacity, recv_x_fp8, recv_scales))) return rc;
    hipError_t err = cgd::launch_layout_and_dispatch_cast_fp8(
        x, num_tokens, hidden, topk_idx, num_topk, num_experts, num_ranks, expert_alignment, scale_format, recv_x_fp8,
        recv_scales, recv_capacity, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank, expert_offset,
        num_recv_tokens_per_expert, recv_src_idx, dst_row, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "layout and FP8 cast dispatch launch");
    return CGD_OK;
}

int cgd_dispatch_cached_fp8(const void* x_fp8, const void* x_scales, int64_t scale_stride_token,
                            int64_t scale_stride_block, int scale_format, int64_t num_tokens, int hidden, int num_topk,
                            const int32_t* dst_row, void* recv_x_fp8, void* recv_scales, int64_t recv_capacity,
                            hipStream_t stream) {
    if (num_tokens < 0) return fail(CGD_ERR_INVALID_ARG, "num_tokens must be >= 0");
    if (num_topk < 1 || num_topk > cgd::kMaxTopk) return fail(CGD_ERR_INVALID_ARG, "num_topk must be in [1,16]");
    int rc = check_fp8(hidden, scale_format);
    if (rc) return rc;
    if (recv_capacity < 0 || recv_capacity > INT32_MAX)
        return fail(CGD_ERR_CAPACITY, "recv_capacity must be in [0, INT32_MAX]");
    if (num_tokens > 0 && (!x_fp8 || !dst_row || (recv_capacity > 0 && !recv_x_fp8)))
        return fail(CGD_ERR_INVALID_ARG, "null pointer");
    if (!aligned(x_fp8, 16) || !aligned(recv_x_fp8, 16))
        return fail(CGD_ERR_INVALID_ARG, "x_fp8 and recv_x_fp8 must be 16-byte aligned");
    if (!aligned(dst_row, 4)) return fail(CGD_ERR_INVALID_ARG, "misaligned dst_row");
    if ((rc = check_scales(x_scales, scale_stride_token, scale_stride_block, scale_format, num_tokens > 0))) return rc;
    if ((rc = check_scales(recv_scales, 0, 0, scale_format, num_tokens > 0 && recv_capacity > 0))) return rc;
    hipError_t err = cgd::launch_dispatch_cached_fp8(x_fp8, x_scales, scale_stride_token, scale_stride_block,
                                                     scale_format, num_tokens, hidden, num_topk, dst_row, recv_x_fp8,
                                                     recv_scales, recv_capacity, stream);
    if (err != hipSuccess) return hip_fail(err, "cached FP8 dispatch launch");
    return CGD_OK;
}

int cgd_normal_dispatch_apply_fp8(const void* x_fp8, const void* x_scales, int64_t scale_stride_token,
                                  int64_t scale_stride_block, int scale_format, int64_t num_tokens, int hidden,
                                  const int64_t* topk_idx, const float* topk_weights, int num_topk, int num_experts,
                                  int num_ranks, void* recv_x_fp8, void* recv_scales, int64_t recv_capacity,
                                  const int32_t* rank_offset, int32_t* recv_src_idx, int32_t* send_row,
                                  int64_t* recv_topk_idx, float* recv_topk_weights, const void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    int rc = check_fp8(hidden, scale_format);
    if (rc) return rc;
    if ((rc = check_normal_apply_args(x_fp8, num_tokens, hidden, topk_idx, topk_weights, num_topk, num_experts,
                                      num_ranks, recv_x_fp8, recv_capacity, rank_offset, recv_src_idx, send_row,
                                      recv_topk_idx, recv_topk_weights, workspace, workspace_bytes)))
        return rc;
    if ((rc = check_scales(x_scales, scale_stride_token, scale_stride_block, scale_format, num_tokens > 0))) return rc;
    if ((rc = check_scales(recv_scales, 0, 0, scale_format, recv_capacity > 0))) return rc;
    hipError_t err = cgd::launch_normal_apply_fp8(x_fp8, x_scales, scale_stride_token, scale_stride_block,
                                                  scale_format, num_tokens, hidden, topk_idx, topk_weights, num_topk,
                                                  num_experts, num_ranks, recv_x_fp8, recv_scales, recv_capacity,
                                                  rank_offset, recv_src_idx, send_row, recv_topk_idx,
                                                  recv_topk_weights, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "FP8 normal dispatch apply launch");
    return CGD_OK;
}

int cgd_normal_dispatch_cached_fp8(const void* x_fp8, const void* x_scales, int64_t scale_stride_token,
                                   int64_t scale_stride_block, int scale_format, int64_t num_tokens, int hidden,
                                   int num_ranks, const int32_t* send_row, void* recv_x_fp8, void* recv_scales,
                                   int64_t recv_capacity, hipStream_t stream) {
    if (num_tokens < 0) return fail(CGD_ERR_INVALID_ARG, "num_tokens must be >= 0");
    if (num_ranks < 1 || num_ranks > cgd::kMaxRanks) return fail(CGD_ERR_INVALID_ARG, "num_ranks must be in [1,384]");
    int rc = check_fp8(hidden, scale_format);
    if (rc) return rc;
    if (recv_capacity < 0 || recv_capacity > INT32_MAX)
        return fail(CGD_ERR_CAPACITY, "recv_capacity must be in [0, INT32_MAX]");
    if (num_tokens > 0 && (!x_fp8 || !send_row || (recv_capacity > 0 && !recv_x_fp8)))
        return fail(CGD_ERR_INVALID_ARG, "null pointer");
    if (!aligned(x_fp8, 16) || !aligned(recv_x_fp8, 16))
        return fail(CGD_ERR_INVALID_ARG, "x_fp8 and recv_x_fp8 must be 16-byte aligned");
    if (!aligned(send_row, 4)) return fail(CGD_ERR_INVALID_ARG, "misaligned send_row");
    if ((rc = check_scales(x_scales, scale_stride_token, scale_stride_block, scale_format, num_tokens > 0))) return rc;
    if ((rc = check_scales(recv_scales, 0, 0, scale_format, num_tokens > 0 && recv_capacity > 0))) return rc;
    hipError_t err = cgd::launch_normal_dispatch_cached_fp8(x_fp8, x_scales, scale_stride_token, scale_stride_block,
                                                            scale_format, num_tokens, hidden, num_ranks, send_row,
                                                            recv_x_fp8, recv_scales, recv_capacity, stream);
    if (err != hipSuccess) return hip_fail(err, "cached FP8 normal dispatch launch");
    return CGD_OK;
}

size_t cgd_packed_workspace_bytes(int64_t num_tokens, int num_topk, int num_experts) {
    // the packed layout has no layout outputs: the per-rank partials are not used
    return cgd_dispatch_workspace_bytes(num_tokens, num_topk, num_experts, 1);
}

static int check_packed_args(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E, int R,
                             int64_t cap, const void* recv_x, const int32_t* count, const int32_t* info,
                             const int32_t* dst_row, const int32_t* stats, const void* workspace,
                             size_t workspace_bytes) {
    int rc = check_routing_sizes(T, K, E, R);
    if (rc) return rc;
    if ((rc = check_hidden(H))) return rc;
    if (cap < 0 || (int64_t)E * cap > INT32_MAX)
        return fail(CGD_ERR_CAPACITY, "expert_capacity must be >= 0 with num_experts * expert_capacity <= INT32_MAX");
    if (!count) return fail(CGD_ERR_INVALID_ARG, "null packed_recv_count");
    if (T > 0 && (!x || !topk_idx || !dst_row)) return fail(CGD_ERR_INVALID_ARG, "null x, topk_idx or dst_row");
    if (cap > 0 && (!recv_x || !info)) return fail(CGD_ERR_INVALID_ARG, "null packed receive pointer");
    if (!aligned(x, 16) || !aligned(recv_x, 16)) return fail(CGD_ERR_INVALID_ARG, "x and packed_recv_x must be 16-byte aligned");
    if (!aligned(topk_idx, 8) || !aligned(count, 4) || !aligned(info, 4) || !aligned(dst_row, 4) || !aligned(stats, 4))
        return fail(CGD_ERR_INVALID_ARG, "misaligned index pointer");
    const size_t need = cgd::dispatch_workspace_bytes(T, K, E, 1);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(CGD_ERR_WORKSPACE, "packed dispatch workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                    workspace_bytes);
    return CGD_OK;
}

int cgd_dispatch_packed(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx, int num_topk,
                        int num_experts, int num_ranks, int64_t expert_capacity, void* packed_recv_x,
                        int32_t* packed_recv_count, int32_t* recv_src_info, int32_t* dst_row,
                        int32_t* cumulative_recv_stats, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = check_packed_args(x, num_tokens, hidden, topk_idx, num_topk, num_experts, num_ranks, expert_capacity,
                               packed_recv_x, packed_recv_count, recv_src_info, dst_row, cumulative_recv_stats,
                               workspace, workspace_bytes);
    if (rc) return rc;
    hipError_t err = cgd::launch_dispatch_packed(x, num_tokens, hidden, topk_idx, num_topk, num_experts,
                                                 (int)expert_capacity, -1, packed_recv_x, nullptr, packed_recv_count,
                                                 recv_src_info, dst_row, cumulative_recv_stats, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "packed dispatch launch");
    return CGD_OK;
}

int cgd_dispatch_packed_cast_fp8(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                 int num_topk, int num_experts, int num_ranks, int64_t expert_capacity,
                                 int scale_format, void* packed_recv_x_fp8, void* packed_recv_scales,
                                 int32_t* packed_recv_count, int32_t* recv_src_info, int32_t* dst_row,
                                 int32_t* cumulative_recv_stats, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    int rc = check_fp8(hidden, scale_format);
    if (rc) return rc;
    if ((rc = check_packed_args(x, num_tokens, hidden, topk_idx, num_topk, num_experts, num_ranks, expert_capacity,
                                packed_recv_x_fp8, packed_recv_count, recv_src_info, dst_row, cumulative_recv_stats,
                                workspace, workspace_bytes)))
        return rc;
    if ((rc = check_scales(packed_recv_scales, 0, 0, scale_format, expert_capacity > 0))) return rc;
    hipError_t err = cgd::launch_dispatch_packed(x, num_tokens, hidden, topk_idx, num_topk, num_experts,
                                                 (int)expert_capacity, scale_format, packed_recv_x_fp8,
                                                 packed_recv_scales, packed_recv_count, recv_src_info, dst_row,
                                                 cumulative_recv_stats, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "packed FP8 dispatch launch");
    return CGD_OK;
}

int cgd_layout_and_dispatch_packed(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                   int num_topk, int num_experts, int num_ranks, int64_t expert_capacity,
                                   void* packed_recv_x, int32_t* packed_recv_count, int32_t* recv_src_info,
                                   int32_t* dst_row, int32_t* cumulative_recv_stats, int32_t* num_tokens_per_rank,
                                   int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    int rc = check_packed_args(x, num_tokens, hidden, topk_idx, num_topk, num_experts, num_ranks, expert_capacity,
                               packed_recv_x, packed_recv_count, recv_src_info, dst_row, cumulative_recv_stats,
                               workspace, workspace_bytes);
    if (rc) return rc;
    if ((rc = check_layout_outputs(num_tokens, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank)))
        return rc;
    if ((rc = check_dispatch_workspace(num_tokens, num_topk, num_experts, num_ranks, workspace, workspace_bytes)))
        return rc;
    hipError_t err = cgd::launch_layout_and_dispatch_packed(
        x, num_tokens, hidden, topk_idx, num_topk, num_experts, num_ranks, (int)expert_capacity, -1, packed_recv_x,
        nullptr, packed_recv_count, recv_src_info, dst_row, cumulative_recv_stats, num_tokens_per_rank,
        num_tokens_per_expert, is_token_in_rank, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "layout and packed dispatch launch");
    return CGD_OK;
}

int cgd_layout_and_dispatch_packed_cast_fp8(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                            int num_topk, int num_experts, int num_ranks, int64_t expert_capacity,
                                            int scale_format, void* packed_recv_x_fp8, void* packed_recv_scales,
                                            int32_t* packed_recv_count, int32_t* recv_src_info, int32_t* dst_row,
                                            int32_t* cumulative_recv_stats, int32_t* num_tokens_per_rank,
                                            int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = check_fp8(hidden, scale_format);
    if (rc) return rc;
    if ((rc = check_packed_args(x, num_tokens, hidden, topk_idx, num_topk, num_experts, num_ranks, expert_capacity,
                                packed_recv_x_fp8, packed_recv_count, recv_src_info, dst_row, cumulative_recv_stats,
                                workspace, workspace_bytes)))
        return rc;
    if ((rc = check_scales(packed_recv_scales, 0, 0, scale_format, expert_capacity > 0))) return rc;
    if ((rc = check_layout_outputs(num_tokens, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank)))
        return rc;
    if ((rc = check_dispatch_workspace(num_tokens, num_topk, num_experts, num_ranks, workspace, workspace_bytes)))
        return rc;
    hipError_t err = cgd::launch_layout_and_dispatch_packed(
        x, num_tokens, hidden, topk_idx, num_topk, num_experts, num_ranks, (int)expert_capacity, scale_format,
        packed_recv_x_fp8, packed_recv_scales, packed_recv_count, recv_src_info, dst_row, cumulative_recv_stats,
        num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank, workspace, stream);
    if (err != hipSuccess) return hip_fail(err, "layout and packed FP8 dispatch launch");
    return CGD_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// cgd_layout_and_dispatch_noalloc: cgd_layout_and_dispatch with its workspace
// in a file-scope device array instead of a buffer of the caller's, for
// callers that cannot allocate. Every GPU the library runs on holds its own
// copy of the array, at its own address, until the process ends; calls on one
// GPU share it, so calls that overlap on one GPU race.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;  // the largest workspace the entry point serves
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];  // device address of `scratch` per device, once set up

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The words of a dispatch workspace that must be zero before its first use
// (the plan's ticket, first in the workspace); every call leaves them zero.
__global__ __launch_bounds__(64) void clear_scratch_ticket(unsigned int* words) { words[threadIdx.x] = 0u; }

// The scratch array's address on the current device. The first call on a
// device looks it up with that device current and enqueues the clearing of
// the ticket words on `stream`, before the work of the call that set it up.
// In host code `scratch` names a host-side stand-in, never the device array:
// only the looked-up address is passed to kernels.
static int scratch_address(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
    if (dev < 0 || dev >= kScratchDevices)
        return fail(CGD_ERR_HIP, "device %d is beyond the %d devices the static scratch serves", dev, kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return hip_fail(err, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(CGD_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
        static_assert(cgd::kTicketBytes == 256, "one wave clears the ticket words");
        hipLaunchKernelGGL(clear_scratch_ticket, dim3(1), dim3(64), 0, stream, static_cast<unsigned int*>(p));
        err = hipGetLastError();
        if (err != hipSuccess) return hip_fail(err, "static scratch set-up launch");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CGD_OK;
}

extern "C" int cgd_layout_and_dispatch_noalloc(const void* x, int64_t num_tokens, int hidden, const int64_t* topk_idx,
                                               int num_topk, int num_experts, int num_ranks, int expert_alignment,
                                               void* recv_x, int64_t recv_capacity, int32_t* num_tokens_per_rank,
                                               int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                                               int32_t* expert_offset, int32_t* num_recv_tokens_per_expert,
                                               int32_t* recv_src_idx, int32_t* dst_row, hipStream_t stream) {
    int rc = check_layout_and_dispatch(x, num_tokens, hidden, topk_idx, num_topk, num_experts, num_ranks,
                                       expert_alignment, recv_x, recv_capacity, num_tokens_per_rank,
                                       num_tokens_per_expert, is_token_in_rank, expert_offset,
                                       num_recv_tokens_per_expert, recv_src_idx, dst_row);
    if (rc) return rc;
    const size_t need = cgd::dispatch_workspace_bytes(num_tokens, num_topk, num_experts, num_ranks);
    if (need > kScratchBytes)
        return fail(CGD_ERR_WORKSPACE,
                    "these sizes need %zu bytes of workspace; the static scratch of "
                    "cgd_layout_and_dispatch_noalloc holds %zu (use cgd_layout_and_dispatch with a workspace)",
                    need, kScratchBytes);
    void* ws = nullptr;
    if ((rc = scratch_address(stream, &ws))) return rc;
    return layout_and_dispatch_launches(x, num_tokens, hidden, topk_idx, num_topk, num_experts, num_ranks,
                                        expert_alignment, recv_x, recv_capacity, num_tokens_per_rank,
                                        num_tokens_per_expert, is_token_in_rank, expert_offset,
                                        num_recv_tokens_per_expert, recv_src_idx, dst_row, ws, stream);
}

// Loads every source file's code object on the current device (the runtime
// loads one on the first use of any of its kernels): hipFuncGetAttributes on
// one kernel of each file. Nothing is allocated or enqueued.
extern "C" int cgd_init(void) {
    hipFuncAttributes a;
    hipError_t err = hipFuncGetAttributes(&a, reinterpret_cast<const void*>(&clear_scratch_ticket));
    if (err == hipSuccess) err = cgd::preload_combine();
    if (err == hipSuccess) err = cgd::preload_copy();
    if (err == hipSuccess) err = cgd::preload_dispatch();
    if (err == hipSuccess) err = cgd::preload_fp8();
    if (err == hipSuccess) err = cgd::preload_normal();
    if (err == hipSuccess) err = cgd::preload_layout();
    if (err != hipSuccess) return hip_fail(err, "loading the GPU code");
    return CGD_OK;
}
