// get_dispatch_layout on gfx950.
//
// Computes, from topk_idx [T,K] (get_dispatch_layout API page, "Return
// Values"): per-expert slot counts, per-rank distinct-token counts and the
// is_token_in_rank matrix. Rank r owns experts [r*L, (r+1)*L) (DeepEP legacy
// test analysis page, low-latency per-expert check).
//
// One launch. Each block takes 256 tokens, one per thread:
//   1. the tile's topk_idx is staged in LDS with coalesced loads;
//   2. each thread adds its slots to an LDS expert histogram and builds the
//      bitmask of ranks its token touches;
//   3. distinct tokens per rank: per wave, one ballot per rank and a popcount
//      of the lanes whose token holds it;
//   4. the tile's is_token_in_rank rows (a contiguous byte range) are written
//      with 16-byte stores;
//   5. blocks publish their partial counts; the last block to finish sums
//      them into the outputs (no pre-zeroed outputs, no second launch).
// The NPU implementation on the API page ("Internal Logic", "Multi-Core
// Strategy") also splits tokens over cores and aggregates partial results
// across cores; here the aggregation is a last-block-done reduction.
//
// NPLAN form: the rank-granular dispatch plan from the same tile (the plan
// needs only is_token_in_rank, which the tile has in registers): the
// per-rank ballots of step 3 are the plan's group words, the tile's per-rank
// counts its tile counts; the last block also turns those into per-tile bases
// and rank offsets and rounds the expert counts up to the alignment.
#include "cgd_device.h"
#include "cgd_launch.h"

namespace cgd {

// Rank-granular plan outputs of the NPLAN form (workspace arrays as the
// rank-granular plan kernel writes them).
struct NormalPlanOut {
    unsigned long long* grp_bal;  // [ceil(T/64), R]
    int32_t* grp_pre;             // [ceil(T/64), R]
    int32_t* tile_base;           // [tiles, R]
    int32_t* rank_offset;         // [R + 1]
    int32_t* nrecv;               // [E] or null
    int A;
};

template <int RW, bool NPLAN = false>  // RW: 64-bit words of the rank mask: 1 (R <= 64) or 6 (R <= 384)
__global__ __launch_bounds__(kLayoutTile) void layout_kernel(const int64_t* __restrict__ topk_idx, int64_t T, int K,
                                                             int E, int R, int L, int32_t* __restrict__ ntpr,
                                                             int32_t* __restrict__ ntpe, uint8_t* __restrict__ itr,
                                                             int32_t* __restrict__ partial,
                                                             unsigned int* __restrict__ ticket, NormalPlanOut np) {
    __shared__ int32_t s_idx[kLayoutTile * kMaxTopk];
    __shared__ uint64_t s_mask[kLayoutTile * RW];
    __shared__ int32_t s_hist[kMaxExperts];
    __shared__ int32_t s_rank[kMaxRanks];
    __shared__ int16_t s_rank_of[kMaxExperts];  // rank owning expert e
    constexpr int kGroups = kLayoutTile / kWave;
    __shared__ uint64_t s_bal[NPLAN ? kGroups * kMaxRanks : 1];
    __shared__ int32_t s_off[NPLAN ? kMaxRanks + 1 : 1];
    __shared__ int32_t s_wsum[kGroups];

    const int tid = threadIdx.x;
    const int lshift = (L & (L - 1)) == 0 ? __builtin_ctz(L) : -1;  // power-of-two experts per rank: a shift
    const int64_t t0 = (int64_t)blockIdx.x * kLayoutTile;
    const int nt = (int)max<int64_t>(0, min<int64_t>(kLayoutTile, T - t0));

    for (int i = tid; i < E; i += kLayoutTile) {
        s_hist[i] = 0;
        s_rank_of[i] = (int16_t)(i / L);
    }
    for (int i = tid; i < R; i += kLayoutTile) s_rank[i] = 0;
    stage_routing<kMaxTopk, kLayoutTile>(topk_idx + t0 * K, nt * K, E, s_idx);
    __syncthreads();

    int e[kMaxTopk];
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) e[k] = (tid < nt && k < K) ? s_idx[tid * K + k] : -1;
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k)
        if (e[k] >= 0) atomicAdd(&s_hist[e[k]], 1);
    uint64_t m[RW];
    token_rank_mask<RW>(e, s_rank_of, lshift, m);
    count_rank_tokens<RW>(m, R, s_rank, s_mask, NPLAN ? s_bal : nullptr);
    __syncthreads();
    // is_token_in_rank rows of this tile: t0*R is a multiple of 16 because
    // kLayoutTile is
    store_token_in_rank<RW, kLayoutTile>(m, s_mask, nt, R, itr + t0 * R);
    if (NPLAN) {
        // the tile's group words and group bases, rank by rank
        const int64_t G = (T + kWave - 1) / kWave;
        for (int r = tid; r < R; r += kLayoutTile) {
            int run = 0;
#pragma unroll
            for (int w = 0; w < kGroups; ++w) {
                const int64_t g = (int64_t)blockIdx.x * kGroups + w;
                const uint64_t b = s_bal[w * R + r];
                if (g < G) {
                    np.grp_bal[g * R + r] = b;
                    np.grp_pre[g * R + r] = run;
                }
                run += __popcll(b);
            }
        }
    }

    if (gridDim.x == 1) {
        for (int i = tid; i < E; i += kLayoutTile) {
            ntpe[i] = s_hist[i];
            if (NPLAN && np.nrecv) np.nrecv[i] = (s_hist[i] + np.A - 1) / np.A * np.A;
        }
        for (int i = tid; i < R; i += kLayoutTile) {
            ntpr[i] = s_rank[i];
            if (NPLAN) np.tile_base[i] = 0;
        }
        if (NPLAN) {
            block_exclusive_scan2(R, [&](int r) { return s_rank[r]; }, s_off, s_wsum);
            __syncthreads();
            for (int r = tid; r <= R; r += kLayoutTile) np.rank_offset[r] = s_off[r];
        }
        return;
    }

    const int W = E + R;
    int32_t* mine = partial + (int64_t)blockIdx.x * W;
    for (int i = tid; i < E; i += kLayoutTile) mine[i] = s_hist[i];
    for (int i = tid; i < R; i += kLayoutTile) mine[E + i] = s_rank[i];
    if (!last_block_done(ticket)) return;

    const int nblk = gridDim.x;
    for (int i = tid; i < W; i += kLayoutTile) {
        // loads issued 16 at a time: few round trips however many blocks
        int s = 0;
        for (int b0 = 0; b0 < nblk; b0 += 16) {
            int v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = (b0 + j < nblk) ? partial[(int64_t)(b0 + j) * W + i] : 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) s += v[j];
        }
        if (i < E) {
            ntpe[i] = s;
            if (NPLAN && np.nrecv) np.nrecv[i] = (s + np.A - 1) / np.A * np.A;
        } else {
            ntpr[i - E] = s;
            if (NPLAN) s_rank[i - E] = s;
        }
    }
    if (NPLAN) {
        // per-tile bases of each rank: running sums down the rank columns
        for (int r = tid; r < R; r += kLayoutTile) {
            int run = 0;
            for (int b0 = 0; b0 < nblk; b0 += 16) {
                int v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = (b0 + j < nblk) ? partial[(int64_t)(b0 + j) * W + E + r] : 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (b0 + j < nblk) np.tile_base[(int64_t)(b0 + j) * R + r] = run;
                    run += v[j];
                }
            }
        }
        __syncthreads();
        block_exclusive_scan2(R, [&](int r) { return s_rank[r]; }, s_off, s_wsum);
        __syncthreads();
        for (int r = tid; r <= R; r += kLayoutTile) np.rank_offset[r] = s_off[r];
    }
    reset_ticket(ticket);
}

int64_t layout_blocks(int64_t T) { return T <= 0 ? 1 : (T + kLayoutTile - 1) / kLayoutTile; }

size_t layout_workspace_bytes(int64_t T, int E, int R) {
    const size_t arr = (size_t)layout_blocks(T) * (size_t)(E + R) * sizeof(int32_t);
    return kTicketBytes + (arr + 255) / 256 * 256;
}

hipError_t launch_layout(const int64_t* topk_idx, int64_t T, int K, int E, int R, int32_t* ntpr, int32_t* ntpe,
                         uint8_t* itr, void* workspace, hipStream_t stream) {
    unsigned int* ticket = reinterpret_cast<unsigned int*>(workspace);
    int32_t* partial = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + kTicketBytes);
    const dim3 grid((unsigned)layout_blocks(T)), block(kLayoutTile);
    const int L = E / R;
    const NormalPlanOut none{nullptr, nullptr, nullptr, nullptr, nullptr, 1};
    if (R <= 64)
        hipLaunchKernelGGL(layout_kernel<1>, grid, block, 0, stream, topk_idx, T, K, E, R, L, ntpr, ntpe, itr,
                           partial, ticket, none);
    else
        hipLaunchKernelGGL(layout_kernel<6>, grid, block, 0, stream, topk_idx, T, K, E, R, L, ntpr, ntpe, itr,
                           partial, ticket, none);
    return hipGetLastError();
}

hipError_t launch_layout_and_normal_plan(const int64_t* topk_idx, int64_t T, int K, int E, int R, int A,
                                         int32_t* ntpr, int32_t* ntpe, uint8_t* itr, int32_t* rank_offset,
                                         int32_t* nrecv, void* workspace, hipStream_t stream) {
    // workspace: the rank-granular plan's workspace (its ticket, at offset 0
    // whatever the sizes, is the one this launch takes), then the block
    // partials
    NormalPlanArrays a = normal_plan_arrays(workspace, T, R);
    unsigned int* ticket = a.ticket;
    int32_t* partial = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + normal_workspace_bytes(T, R));
    const dim3 grid((unsigned)layout_blocks(T)), block(kLayoutTile);
    const NormalPlanOut np{a.grp_bal, a.grp_pre, a.tile_base, rank_offset, nrecv, A};
    const int L = E / R;
    if (R <= 64)
        hipLaunchKernelGGL((layout_kernel<1, true>), grid, block, 0, stream, topk_idx, T, K, E, R, L, ntpr, ntpe, itr,
                           partial, ticket, np);
    else
        hipLaunchKernelGGL((layout_kernel<6, true>), grid, block, 0, stream, topk_idx, T, K, E, R, L, ntpr, ntpe, itr,
                           partial, ticket, np);
    return hipGetLastError();
}

}  // namespace cgd
