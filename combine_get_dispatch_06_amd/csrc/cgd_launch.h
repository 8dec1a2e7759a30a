// Internal launchers of libcgd (host side). Arguments are validated by the
// C-ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cgd {

// Size limits of the get_dispatch_layout API ("Parameters", "Notes").
constexpr int kMaxTopk = 16;
constexpr int kMaxExperts = 512;
constexpr int kMaxRanks = 384;

// Tokens per block of the layout kernel and per tile of the dispatch ranking.
constexpr int kLayoutTile = 256;
constexpr int kRankTile = 256;
constexpr size_t kTicketBytes = 256;  // ticket word, padded to keep arrays 256-B aligned

// Work-item ids of a launch are 32-bit: grids of 64-lane waves stay within
// 2^31 work-items, and kernels with a wave per (token, chunk) are issued over
// token ranges of at most this many tokens.
constexpr int64_t kMaxGridWaves = int64_t(1) << 25;
inline int64_t tokens_per_launch(int64_t waves_per_token) {
    return waves_per_token <= 0 ? kMaxGridWaves : (kMaxGridWaves / waves_per_token > 0 ? kMaxGridWaves / waves_per_token : 1);
}

int64_t layout_blocks(int64_t T);
size_t layout_workspace_bytes(int64_t T, int E, int R);
size_t dispatch_workspace_bytes(int64_t T, int K, int E);

hipError_t launch_layout(const int64_t* topk_idx, int64_t T, int K, int E, int R, int32_t* ntpr, int32_t* ntpe,
                         uint8_t* itr, void* workspace, hipStream_t stream);

// Batches of at most one plan tile: plan and apply (bf16) in one launch.
bool dispatch_fuses(int64_t T);
hipError_t launch_dispatch_fused(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E, int A,
                                 void* recv_x, int64_t cap, int32_t* expert_offset, int32_t* recv_src_idx,
                                 int32_t* dst_row, void* workspace, hipStream_t stream);
// The same with get_dispatch_layout's outputs from the same launch.
hipError_t launch_layout_and_dispatch_fused(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E,
                                            int R, int A, void* recv_x, int64_t cap, int32_t* ntpr, int32_t* ntpe,
                                            uint8_t* itr, int32_t* expert_offset, int32_t* recv_src_idx,
                                            int32_t* dst_row, void* workspace, hipStream_t stream);

// The rank-granular plan's workspace arrays (group words, group bases, tile
// counts / bases), as launch_normal_plan leaves them.
struct NormalPlanArrays {
    unsigned int* ticket;  // at offset 0: a ticket of this workspace never moves with the sizes
    unsigned long long* grp_bal;
    int32_t* grp_pre;
    int32_t* tile_base;
};
NormalPlanArrays normal_plan_arrays(void* workspace, int64_t T, int R);

// get_dispatch_layout and the rank-granular dispatch plan in one launch; the
// workspace holds the plan's workspace followed by the layout's.
hipError_t launch_layout_and_normal_plan(const int64_t* topk_idx, int64_t T, int K, int E, int R, int A,
                                         int32_t* ntpr, int32_t* ntpe, uint8_t* itr, int32_t* rank_offset,
                                         int32_t* nrecv, void* workspace, hipStream_t stream);

// The dispatch plan: the handle (expert_offset, recv_src_idx, dst_row) from
// the routing alone.
hipError_t launch_dispatch_plan(const int64_t* topk_idx, int64_t T, int K, int E, int A, int64_t cap,
                                int32_t* expert_offset, int32_t* recv_src_idx, int32_t* dst_row, void* workspace,
                                hipStream_t stream);

// get_dispatch_layout and the dispatch plan from one pass over the routing.
hipError_t launch_layout_and_plan(const int64_t* topk_idx, int64_t T, int K, int E, int R, int A, int64_t cap,
                                  int32_t* ntpr, int32_t* ntpe, uint8_t* itr, int32_t* expert_offset,
                                  int32_t* recv_src_idx, int32_t* dst_row, void* workspace, hipStream_t stream);

// Packed fixed-capacity layout: plan + apply; fmt < 0 moves bf16 rows, else
// casts to FP8 with that scale format.
hipError_t launch_dispatch_packed(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E,
                                  int expert_capacity, int fmt, void* recv_x, void* recv_s, int32_t* packed_count,
                                  int32_t* recv_src_info, int32_t* dst_row, int32_t* stats, void* workspace,
                                  hipStream_t stream);

hipError_t launch_dispatch_cached(const void* x, int64_t T, int H, int K, const int32_t* dst_row, void* recv_x,
                                  int64_t cap, hipStream_t stream);

hipError_t launch_combine(const void* expert_out, int64_t cap, int H, const int32_t* dst_row, const float* w,
                          int64_t T, int K, void* out, hipStream_t stream);

size_t normal_workspace_bytes(int64_t T, int R);

hipError_t launch_normal_plan(const uint8_t* itr, int64_t T, int R, const int32_t* ntpe, int E, int A,
                              int32_t* rank_offset, int32_t* nrecv, void* workspace, hipStream_t stream);

hipError_t launch_normal_apply(const void* x, int64_t T, int H, const int64_t* topk_idx, const float* topk_w, int K,
                               int E, int R, void* recv_x, int64_t cap, const int32_t* rank_offset,
                               int32_t* recv_src_idx, int32_t* send_row, int64_t* recv_topk_idx, float* recv_topk_w,
                               const void* workspace, hipStream_t stream);

hipError_t launch_normal_dispatch_cached(const void* x, int64_t T, int H, int R, const int32_t* send_row,
                                         void* recv_x, int64_t cap, hipStream_t stream);

hipError_t launch_normal_combine(const void* expert_out, int64_t rows, int H, const int32_t* send_row, int64_t T,
                                 int R, const float* recv_w, int K, const void* bias0, const void* bias1, void* out,
                                 float* out_w, hipStream_t stream);

// FP8 payload (scale format 0 fp32, 1 fp32 power of two, 2 UE8M0 byte).
hipError_t launch_cast_to_fp8(const void* x, int64_t T, int H, void* q, void* scales, int64_t st, int64_t sb, int fmt,
                              hipStream_t stream);

// Plain 16-byte copy of `bytes` (a multiple of 16).
hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

hipError_t launch_cast_back(const void* q, const void* scales, int64_t st, int64_t sb, int fmt, int64_t T, int H,
                            void* out, hipStream_t stream);

// Cast to FP8 on the way: bf16 x moved to the rows of a handle's dst_row as
// e4m3 codes and per-block scales.
hipError_t launch_dispatch_cached_cast_fp8(const void* x, int64_t T, int H, int K, int fmt, const int32_t* dst_row,
                                           void* recv_q, void* recv_s, int64_t cap, hipStream_t stream);

hipError_t launch_dispatch_cached_fp8(const void* xq, const void* xs, int64_t st, int64_t sb, int fmt, int64_t T,
                                      int H, int K, const int32_t* dst_row, void* recv_q, void* recv_s, int64_t cap,
                                      hipStream_t stream);

hipError_t launch_normal_apply_fp8(const void* xq, const void* xs, int64_t st, int64_t sb, int fmt, int64_t T, int H,
                                   const int64_t* topk_idx, const float* topk_w, int K, int E, int R, void* recv_q,
                                   void* recv_s, int64_t cap, const int32_t* rank_offset, int32_t* recv_src_idx,
                                   int32_t* send_row, int64_t* recv_topk_idx, float* recv_topk_w,
                                   const void* workspace, hipStream_t stream);

hipError_t launch_normal_dispatch_cached_fp8(const void* xq, const void* xs, int64_t st, int64_t sb, int fmt,
                                             int64_t T, int H, int R, const int32_t* send_row, void* recv_q,
                                             void* recv_s, int64_t cap, hipStream_t stream);

}  // namespace cgd
