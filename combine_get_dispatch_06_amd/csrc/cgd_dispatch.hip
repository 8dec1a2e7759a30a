// Dispatch permutation on gfx950.
//
// Every selected (token, slot) pair gets one row of its expert's receive
// segment; segments are laid end to end in ascending expert id, each sized to
// its row count rounded up to expert_alignment (DeepEP Python interface notes,
// "Dispatch API": expert_alignment, the receive buffer and the handle). Inside
// a segment, rows follow ascending (token, slot), which makes the permutation
// unique and independent of scheduling.
//
// No block ever waits for another. The plan needs only the routing and
// writes the whole handle; the apply only moves rows.
//   rank_kernel     (the plan) one block per tile of 256 tokens (4 waves, one
//                   token per lane). For each slot it finds the number of
//                   earlier slots of the tile with the same expert. When no
//                   token of the tile repeats an expert, each wave sets one
//                   bit per (expert, lane) in a 64-bit LDS mask per expert;
//                   the rank is the popcount of the mask below the lane plus
//                   the rows of earlier waves. Otherwise it counts slot by slot
//                   with wavefront ballots (a "multi-split" over the bits of
//                   the expert id). It writes a packed (expert, rank-in-tile)
//                   word per slot and the tile's expert histogram. The last
//                   block to finish turns the histograms into per-tile bases
//                   (rows of the expert in earlier tiles, one pass), the
//                   per-expert counts and the segment offsets: a block prefix
//                   scan of the aligned counts, or e * capacity for the
//                   fixed-capacity packed layout. A one-tile grid finishes
//                   from LDS without the handshake and writes dst_row and
//                   recv_src_idx itself. Its LAYOUT form also writes
//                   get_dispatch_layout's outputs from the same tile.
//   finalize_kernel the plan's last step for several tiles: one thread per
//                   slot turns its packed word into the final row (segment
//                   offset + tile base + rank) and records dst_row and
//                   recv_src_idx; rows without data get recv_src_idx = -1
//                   (padding, unused capacity, tail).
//   the apply       moves each row to its final rows, reading it from HBM
//                   once however many experts it goes to. Batches of >= 16384
//                   slots: scatter_kernel, one wave per (token, U KB chunk,
//                   group of S slots), the chunk's K/S waves adjacent so that
//                   they share its load through L2. Smaller batches:
//                   scatter_bcast_kernel, one wave per (token, chunk) stores
//                   the chunk to each of the K rows. scatter_cast_kernel is
//                   the FP8 form (cast on the way, one wave per chunk).
//                   Cached dispatch is the same apply on a stored dst_row.
//   FUSED           batches of at most one tile (decode) through cgd_dispatch
//                   or the bf16 packed dispatch: rank_kernel plans and moves
//                   the rows in one launch (every block plans the batch).
//
// Measured on MI355X: the receive layout bounds the apply. The same 16-byte
// copy writes token-major destinations (token t's K rows side by side) about
// 20 % faster than the expert-major rows the method prescribes, at hidden
// 7168 whatever the grouping of rows up to 896 KB; the apply runs within a
// few % of the latter. Each wave's rows come after one dependent load (hence
// the final rows from the plan), and x arrives from HBM into waves that wait
// for it, which slot groups and the plan's prefetch of x hide. Destination-
// ordered copies (sequential stores) lose more on the 8x scattered re-reads
// of x than they gain.
#include <algorithm>
#include <atomic>

#include "cgd_device.h"
#include "cgd_launch.h"

namespace cgd {

constexpr int kRankWaves = kRankTile / kWave;
constexpr int kPackBits = 13;  // rank inside a tile < 256 * 16 = 4096 < 2^13
constexpr int kScatterWaves = 4;  // waves per block of the broadcast and cast-on-dispatch kernels
constexpr int kSlotWaves = 16;    // waves per block of the row copy
constexpr int kBatch = 16;                        // loads in flight per thread when summing columns

// LDS of the rank kernel, carved from dynamic shared memory sized for (E, K).
size_t rank_lds_bytes(int E, int K) {
    return (size_t)kRankWaves * E * 8      // tok: lanes of a wave holding expert e
           + (size_t)kRankWaves * E * 4    // pre: rows of expert e in earlier waves of the tile
           + (size_t)kRankTile * K * 4     // slot: routing of the tile, then packed rows
           + (size_t)(E + 1) * 4           // off: segment offsets (last block)
           + kRankWaves * 4 + 16;          // wsum
}

// Expert of a slot word during the duplicate-aware count (-1: not selected).
__device__ __forceinline__ int slot_expert(int v) { return v < 0 ? -1 : (v & 0xFFFF); }

// recv_src_idx = -1 for every row that holds no data: rows of segment e past
// its count (alignment padding, unused fixed capacity) and rows past the last
// segment. Threads are spread over (segment, row) pairs, so each thread needs
// only its segment's bounds, whatever the grid size.
__device__ __forceinline__ void fill_unused(int32_t* __restrict__ recv_src_idx,
                                            const int32_t* __restrict__ expert_offset,
                                            const int32_t* __restrict__ counts, int E, int64_t cap, uint32_t gid,
                                            uint32_t nth) {
    // 32-bit arithmetic: rows < cap <= INT32_MAX, thread ids < 2^32
    const uint32_t end = (uint32_t)max<int64_t>(0, min<int64_t>(expert_offset[E], cap));
    if (nth >= (uint32_t)E) {
        const uint32_t per = nth / (uint32_t)E;  // threads per segment
        const uint32_t seg = gid / per;
        if (seg < (uint32_t)E) {
            const uint32_t lo = (uint32_t)max(0, expert_offset[seg] + max(counts[seg], 0));
            const uint32_t hi = (uint32_t)max<int64_t>(0, min<int64_t>(expert_offset[seg + 1], end));  // <= cap
            for (uint32_t r = lo + (gid - seg * per); r < hi; r += per) recv_src_idx[r] = -1;
        }
    } else {
        for (uint32_t e = gid; e < (uint32_t)E; e += nth) {
            const uint32_t lo = (uint32_t)max(0, expert_offset[e] + max(counts[e], 0));
            const uint32_t hi = (uint32_t)max<int64_t>(0, min<int64_t>(expert_offset[e + 1], end));
            for (uint32_t r = lo; r < hi; ++r) recv_src_idx[r] = -1;
        }
    }
    for (int64_t r = (int64_t)end + gid; r < cap; r += nth) recv_src_idx[r] = -1;
}

// The first kFillThreads threads of a grid of BLOCK-thread blocks (all of a
// smaller grid) do the fill: each filling wave reads the same few lines of
// expert_offset and counts, so only as many waves as the fill needs take
// part (the rows of a large fixed capacity are then several per thread).
constexpr int kFillThreads = 32768;

template <int BLOCK>
__device__ __forceinline__ void fill_unused_grid(int32_t* __restrict__ recv_src_idx,
                                                 const int32_t* __restrict__ expert_offset,
                                                 const int32_t* __restrict__ counts, int E, int64_t cap) {
    const int nb = min((int)gridDim.x, kFillThreads / BLOCK);
    if ((int)blockIdx.x >= nb) return;
    fill_unused(recv_src_idx, expert_offset, counts, E, cap, blockIdx.x * BLOCK + threadIdx.x, (uint32_t)nb * BLOCK);
}

struct LayoutOut {
    int R, L;
    int32_t* ntpr;
    int32_t* ntpe;
    uint8_t* itr;
    int32_t* rank_part;
};

// Outputs of a one-tile batch, which is planned from LDS alone: the handle
// (dst_row, recv_src_idx, rows below cap) and, in the FUSED form, the row
// copy: the grid's waves take the (token, 1 KB chunk) items of x in turn, at
// most kFusedItems each, and move them to the tokens' receive rows.
constexpr int kFusedItems = 4;
struct TileOut {
    int32_t* dst_row;
    int32_t* recv_src_idx;
    int64_t cap;
    const uint4* x;  // FUSED only
    int nvec, nchunk;
    uint4* recv_x;
    // FUSED with CAST: the rows receive x's FP8 codes (nvec 8-byte vectors
    // per row, rq) and scales (nsb per row, rs: fp32, or a UE8M0 byte for
    // fmt 2) in place of the bf16 rows
    int fmt, nsb;
    uint2* rq;
    void* rs;
};

// rank_kernel. Slot loops read the routing from LDS, which keeps the kernel
// light on registers for any num_topk. seg_cap >= 0 selects the
// fixed-capacity packed layout: segment e is rows [e*seg_cap, (e+1)*seg_cap)
// whatever its count (seg_cap < 0: prefix-summed segments of the aligned
// counts). counts receives every expert's slot count (workspace, for the -1
// fill); packed_count (min(count, seg_cap)) and stats (accumulates
// packed_count) are optional. With LAYOUT the kernel also produces
// get_dispatch_layout's outputs from the same staged tile (rank masks with RW
// 64-bit words, as the layout kernel): is_token_in_rank rows per tile,
// per-tile distinct-token counts per rank (rank_part, workspace) summed by
// the last block into ntpr, and ntpe = the column totals of the tile
// histograms.
//
// A batch of one tile (decode) finishes from LDS: the kernel writes the
// final dst_row and recv_src_idx itself and fills the unused rows. FUSED:
// every block plans the whole batch in LDS (a few microseconds of LDS work,
// cheaper than a second launch and a second pass over the plan), block 0
// alone computes and writes the plan's and the layout's outputs, every block
// fills a share of the unused rows, and each wave of blocks 1.. (of block 0
// too when it is alone) then moves up to kFusedItems (token, chunk) items to
// the tokens' rows, their x chunks loaded once the routing is staged (none
// with nvec = 0: the plan alone of a one-tile batch with many spare rows).
// Lanes without a token skip the LDS mask atomics. Larger batches
// leave packed slot words and tile bases in the workspace for
// finalize_kernel; blocks past the plan_tiles tiles (if any) prefetch x
// (px, pvecs 16-byte vectors) and take no part in the plan. FUSED with CAST:
// each item's chunk is cast to FP8 as the per-token cast does (a 16-lane
// group holds one 128-channel block) and its codes and scales go to the rows.
template <int RW, bool LAYOUT, bool FUSED = false, bool CAST = false>
__global__ __launch_bounds__(kRankTile) void rank_kernel(const int64_t* __restrict__ topk_idx, int64_t T, int K, int E,
                                                         int ebits, int A, int seg_cap, int32_t* __restrict__ slot_pack,
                                                         int32_t* __restrict__ tile_base,
                                                         int32_t* __restrict__ expert_offset,
                                                         int32_t* __restrict__ nrecv,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ packed_count,
                                                         int32_t* __restrict__ stats,
                                                         unsigned int* __restrict__ ticket, LayoutOut lo,
                                                         TileOut fc, int plan_tiles, const uint4* __restrict__ px,
                                                         int64_t pvecs) {
    if (!FUSED && (int)blockIdx.x >= plan_tiles) {
        prefetch_rows<kRankTile>(px, pvecs, (int)blockIdx.x - plan_tiles, (int)gridDim.x - plan_tiles);
        return;
    }
    extern __shared__ __align__(16) char lds[];
    unsigned long long* s_tok = reinterpret_cast<unsigned long long*>(lds);
    int32_t* s_pre = reinterpret_cast<int32_t*>(s_tok + kRankWaves * E);
    int32_t* s_slot = s_pre + kRankWaves * E;
    int32_t* s_off = s_slot + kRankTile * K;
    int32_t* s_wsum = s_off + E + 1;
    const int tile = FUSED ? 0 : blockIdx.x;
    const int ntiles = FUSED ? 1 : plan_tiles;
    const bool writer = !FUSED || blockIdx.x == 0;  // writes the plan's outputs
    // FUSED: the blocks before m0 move no rows; block 0 writes the plan's
    // outputs and, in a grid of three or more, block 1 the layout's (else
    // block 0 both)
    const unsigned m0 = !FUSED ? 0u : gridDim.x > 2 && LAYOUT ? 2u : gridDim.x > 1 ? 1u : 0u;
    const bool lwriter = !FUSED || blockIdx.x == (m0 == 2 ? 1u : 0u);  // writes the layout's outputs

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = lane_id();
    const int64_t t0 = (int64_t)tile * kRankTile;
    const int nt = (int)max<int64_t>(0, min<int64_t>(kRankTile, T - t0));

    // FUSED: this wave's (token, chunk) items (a batch of at most one tile:
    // item numbers fit in 32 bits). The blocks that alone compute and write
    // the plan's and the layout's outputs move no rows: the others' items
    // end about when they do.
    int64_t ft[kFusedItems];
    int fv[kFusedItems];
    if (FUSED) {
        const unsigned nbm = gridDim.x - m0;  // blocks m0.. move the rows
        const unsigned w0 = (blockIdx.x >= m0 ? blockIdx.x - m0 : 0u) * kRankWaves +
                            __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
        for (int j = 0; j < kFusedItems; ++j) {
            unsigned item = w0 + (unsigned)j * nbm * kRankWaves;
            if (blockIdx.x < m0) item = 0xFFFFFFF0u;  // no items: ft >= T below
            const unsigned tj = item / (unsigned)fc.nchunk;
            ft[j] = tj;
            fv[j] = (int)(item - tj * (unsigned)fc.nchunk) * kWave + lane;
        }
    }
    // top-k <= kDirectTopk: this thread's token's routing straight into
    // registers, in flight across the barrier that orders the LDS set-up
    // (the tile's routing reaches LDS from registers below, for the phases
    // that read other tokens' slots); larger top-k: the coalesced stage
    const bool direct = K <= kDirectTopk;
    int64_t raw[kMaxTopk];
    {
        const int64_t* tok = topk_idx + (t0 + min(tid, max(nt - 1, 0))) * K;
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k) raw[k] = (direct && tid < nt && k < K) ? tok[k] : -1;
    }
    for (int i = tid; i < kRankWaves * E; i += kRankTile) {
        s_tok[i] = 0ull;
        s_pre[i] = 0;
    }
    __shared__ uint64_t s_mask[LAYOUT ? kRankTile * RW : 1];
    __shared__ int32_t s_rank[LAYOUT ? kMaxRanks : 1];
    __shared__ int16_t s_rank_of[LAYOUT ? kMaxExperts : 1];
    if (LAYOUT) {
        for (int i = tid; i < E; i += kRankTile) s_rank_of[i] = (int16_t)(i / lo.L);
        for (int i = tid; i < lo.R; i += kRankTile) s_rank[i] = 0;
    }
    if (!direct) stage_routing<kMaxTopk, kRankTile>(topk_idx + t0 * K, nt * K, E, s_slot);
    __syncthreads();
    // FUSED: this wave's items, their x chunks loaded now, after the stage:
    // loads complete in issue order, so x loads issued before the routing
    // would hold up the stage; the plan's LDS work hides them (the item
    // indexes were computed while the routing loads were in flight)
    uint4 fbuf[kFusedItems];
    if (FUSED) {
#pragma unroll
        for (int j = 0; j < kFusedItems; ++j) {
            fbuf[j] = make_uint4(0, 0, 0, 0);
            if (ft[j] < T && fv[j] < fc.nvec) fbuf[j] = fc.x[ft[j] * fc.nvec + fv[j]];
        }
    }

    int32_t* my = s_slot + tid * K;  // this token's K slots
    const bool mine = tid < nt;
    const uint64_t lt = lanemask_lt();
    const uint64_t bit = 1ull << lane;
    int e[kMaxTopk];
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
        if (direct)
            e[k] = (raw[k] >= 0 && raw[k] < E) ? (int)raw[k] : -1;
        else
            e[k] = (mine && k < K) ? my[k] : -1;
    }
    if (direct && mine)
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k)
            if (k < K) my[k] = e[k];

    // ---- 1. rank of every slot inside the tile; tile histogram ----
    // Each wave sets one bit per (expert, lane) in a 64-bit LDS mask per
    // expert. The previous mask returned by the atomic also tells whether this
    // token already holds the expert in an earlier slot.
    // all K atomics are issued before any result is used; the results follow
    // together. Lanes without a selected expert (no token: the idle waves of
    // a short tile) take no part: as dummy operations on one common word
    // they would be a 64-way same-address LDS atomic each (about 2 us at
    // decode).
    uint64_t prev[kMaxTopk];
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
        prev[k] = 0;
        if (k < K && e[k] >= 0) prev[k] = atomicOr(&s_tok[wave * E + e[k]], bit);
    }
    bool dup = false;
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) dup |= e[k] >= 0 && (prev[k] & bit) != 0;
    uint64_t m[RW];
    if (LAYOUT && lwriter) {  // FUSED: only one block writes the layout outputs
        const int lshift = (lo.L & (lo.L - 1)) == 0 ? __builtin_ctz(lo.L) : -1;
        token_rank_mask<RW>(e, s_rank_of, lshift, m);
        count_rank_tokens<RW>(m, lo.R, s_rank, s_mask);
    }
    const bool any_dup = __syncthreads_or(dup);
    if (LAYOUT && lwriter) {
        // t0*R is a multiple of 16 because kRankTile is
        store_token_in_rank<RW, kRankTile>(m, s_mask, nt, lo.R, lo.itr + t0 * lo.R);
        for (int r = tid; r < lo.R; r += kRankTile) lo.rank_part[(int64_t)tile * lo.R + r] = s_rank[r];
    }
    if (!any_dup) {
        // Every token holds an expert at most once: the rank of (t,k) among
        // the tile's rows of expert e is the number of earlier tokens holding
        // e: the lanes below mine in my wave's mask plus earlier waves' rows.
        for (int x = tid; x < E; x += kRankTile) {
            uint64_t mk[kRankWaves];  // all mask reads before any store (same LDS array)
#pragma unroll
            for (int w = 0; w < kRankWaves; ++w) mk[w] = s_tok[w * E + x];
            int run = 0;
#pragma unroll
            for (int w = 0; w < kRankWaves; ++w) {
                s_pre[w * E + x] = run;
                run += __popcll(mk[w]);
            }
            if (ntiles > 1) tile_base[(int64_t)tile * E + x] = run;
            s_off[x] = run;  // the tile's histogram (one-tile grids finish from it)
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k)
            if (e[k] >= 0)
                my[k] = (e[k] << kPackBits) | (s_pre[wave * E + e[k]] + __popcll(s_tok[wave * E + e[k]] & lt));
    } else {
        // Some token repeats an expert: count slot by slot. Lanes whose k'-th
        // expert agrees with my k-th expert on every bit of the expert id are
        // its peers in column k' ("multi-split" ballots); peers below my lane
        // plus my own earlier equal slots give the rank inside the wave. Until
        // the wave prefixes are known a slot word holds expert | rank << 16.
        for (int k = 0; k < K; ++k) {
            const int e = mine ? slot_expert(my[k]) : -1;
            int rk = 0;
            for (int kp = 0; kp < K; ++kp) {
                const int ep = mine ? slot_expert(my[kp]) : -1;
                uint64_t peers = ballot(ep >= 0);
                for (int b = 0; b < ebits; ++b) {
                    const uint64_t col = ballot((ep >> b) & 1);
                    peers &= ((e >> b) & 1) ? col : ~col;
                }
                rk += __popcll(peers & lt) + ((kp < k && ep == e) ? 1 : 0);
            }
            if (e >= 0) {
                atomicAdd(&s_pre[wave * E + e], 1);
                my[k] = e | (rk << 16);
            }
        }
        __syncthreads();
        for (int x = tid; x < E; x += kRankTile) {
            int run = 0;
#pragma unroll
            for (int w = 0; w < kRankWaves; ++w) {
                const int c = s_pre[w * E + x];
                s_pre[w * E + x] = run;
                run += c;
            }
            if (ntiles > 1) tile_base[(int64_t)tile * E + x] = run;
            s_off[x] = run;
        }
        __syncthreads();
        if (mine)
            for (int k = 0; k < K; ++k) {
                const int v = my[k];
                if (v >= 0) {
                    const int e = v & 0xFFFF;
                    my[k] = (e << kPackBits) | ((v >> 16) + s_pre[wave * E + e]);
                }
            }
    }

    __syncthreads();
    if (ntiles > 1) {
        int32_t* out = slot_pack + t0 * K;
        const int n = nt * K;
        for (int i = tid; i < n; i += kRankTile) out[i] = s_slot[i];
    }

    if (ntiles == 1) {
        // one tile (decode batches): its histogram, in LDS, is the total and
        // no other block has to be waited for
        for (int x = tid; x < E; x += kRankTile) {
            s_pre[x] = s_off[x];
            if (LAYOUT && lwriter) lo.ntpe[x] = s_off[x];
        }
        if (LAYOUT && lwriter)
            for (int r = tid; r < lo.R; r += kRankTile) lo.ntpr[r] = s_rank[r];
    } else {
    if (!last_block_done(ticket, ntiles)) return;

    // ---- 2. last block: per-tile bases and segment offsets ----
    // one pass over the tile histograms: each becomes the rows of its expert
    // in earlier tiles (the apply adds the segment offset), and the column
    // total is the expert's row count
    for (int x = tid; x < E; x += kRankTile) {
        int run = 0;
        for (int b0 = 0; b0 < ntiles; b0 += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) v[j] = (b0 + j < ntiles) ? tile_base[(int64_t)(b0 + j) * E + x] : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (b0 + j < ntiles) tile_base[(int64_t)(b0 + j) * E + x] = run;
                run += v[j];
            }
        }
        s_pre[x] = run;
    }
    if (LAYOUT) {
        // layout outputs: slot totals per expert, distinct tokens per rank
        for (int x = tid; x < E; x += kRankTile) lo.ntpe[x] = s_pre[x];
        for (int r = tid; r < lo.R; r += kRankTile) {
            int run = 0;
            for (int b0 = 0; b0 < ntiles; b0 += kBatch) {
                int v[kBatch];
#pragma unroll
                for (int j = 0; j < kBatch; ++j)
                    v[j] = (b0 + j < ntiles) ? lo.rank_part[(int64_t)(b0 + j) * lo.R + r] : 0;
#pragma unroll
                for (int j = 0; j < kBatch; ++j) run += v[j];
            }
            lo.ntpr[r] = run;
        }
    }
    reset_ticket(ticket);
    }
    __syncthreads();
    if (seg_cap >= 0) {
        // fixed-capacity segments
        for (int x = tid; x <= E; x += kRankTile) s_off[x] = x * seg_cap;
        for (int x = tid; x < E && writer; x += kRankTile) {
            const int placed = min(s_pre[x], seg_cap);
            if (packed_count) packed_count[x] = placed;
            if (stats) stats[x] += placed;
        }
    } else {
        // segment offsets: exclusive scan of the aligned sizes
        block_exclusive_scan2(E, [&](int x) { return (s_pre[x] + A - 1) / A * A; }, s_off, s_wsum);
    }
    __syncthreads();
    if (writer) {
        for (int x = tid; x < E; x += kRankTile) {
            counts[x] = s_pre[x];
            if (nrecv) nrecv[x] = (s_pre[x] + A - 1) / A * A;  // aligned segment size
        }
        for (int x = tid; x <= E; x += kRankTile) expert_offset[x] = s_off[x];
    }
    if (ntiles > 1) return;  // finalize_kernel completes the handle

    // ---- one tile: final rows and unused rows; FUSED: this wave's items ----
    // The final row of a packed (expert, rank) word: segment offset + rank,
    // or the fixed-capacity row; -1 past the capacity or the buffer.
    auto row_of = [&](int v) {
        if (v < 0) return -1;
        const int ex = v >> kPackBits, r = v & ((1 << kPackBits) - 1);
        const int d = seg_cap >= 0 ? (r < seg_cap ? ex * seg_cap + r : -1) : s_off[ex] + r;
        return d < fc.cap ? d : -1;
    };
    // the block that writes the handle turns every slot word into its row;
    // the other blocks of a FUSED grid resolve only their items' rows, below
    const bool all_rows = !FUSED || writer;
    if (mine && all_rows) {
        for (int k = 0; k < K; ++k) {
            const int d = row_of(my[k]);
            my[k] = d;
            if (writer) {
                fc.dst_row[(int64_t)tid * K + k] = d;
                if (d >= 0) fc.recv_src_idx[d] = tid;
            }
        }
    }
    fill_unused(fc.recv_src_idx, s_off, s_pre, E, fc.cap, blockIdx.x * kRankTile + tid, gridDim.x * kRankTile);
    if (!FUSED) return;
    if (all_rows) __syncthreads();  // the moves below read the rows just written
#pragma unroll
    for (int j = 0; j < kFusedItems; ++j) {
        if (ft[j] < T) {  // wave-uniform
            int dl = -1;
            if (lane < K) {
                const int v = s_slot[ft[j] * K + lane];
                dl = all_rows ? v : row_of(v);
            }
            const bool in = fv[j] < fc.nvec;  // with CAST whole 16-lane groups are in or out (H % 128 == 0)
            uint2 code = make_uint2(0, 0);
            Fp8Scale sc{0.0f, 0.0f, 0u};
            if (CAST) {
                sc = fp8_block_scale(group16_max(in ? absmax_bf16x8(fbuf[j]) : 0.0f), fc.fmt);
                code = quantize_bf16x8(fbuf[j], sc.mul);
            }
            for (int k = 0; k < K; ++k) {
                const int d = __builtin_amdgcn_readlane(dl, k);
                if (d < 0 || !in) continue;
                if (CAST) {
                    store_nt(fc.rq + (int64_t)d * fc.nvec + fv[j], code);
                    if ((lane & 15) == 0) {
                        const int64_t si = (int64_t)d * fc.nsb + fv[j] / 16;
                        if (fc.fmt == 2)
                            static_cast<uint8_t*>(fc.rs)[si] = (uint8_t)sc.ue8m0;
                        else
                            static_cast<float*>(fc.rs)[si] = sc.scale;
                    }
                } else {
                    store_nt(fc.recv_x + (int64_t)d * fc.nvec + fv[j], fbuf[j]);
                }
            }
        }
    }
}

// Final receive row of a packed slot word p from the plan (-1: not selected).
// A consistent plan gives an expert < E and a row inside the expert's segment
// and below cap; anything else maps to -1 (a slot past a fixed capacity is
// dropped), so no access leaves the workspace or the receive buffer.
__device__ __forceinline__ int final_row(int p, int64_t t, const int32_t* __restrict__ tile_base, int E,
                                         const int32_t* __restrict__ expert_offset, int64_t cap) {
    // the three loads are independent (the expert is clamped into range for
    // them), so they are issued together
    const int ex = p >> kPackBits;
    const int exc = min(max(ex, 0), E - 1);
    const int lo = expert_offset[exc], hi = expert_offset[exc + 1];
    const int tb = tile_base[(t / kRankTile) * E + exc];
    const int d = lo + tb + (p & ((1 << kPackBits) - 1));
    return (p < 0 || ex >= E || d < 0 || d >= cap || d >= hi) ? -1 : d;
}

// Final rows of every slot of a batch of several tiles (the plan's last
// step): one thread per (token, slot) turns the packed word into the receive
// row (segment offset + tile base + rank) and records dst_row and
// recv_src_idx; the first kFillThreads threads then fill unused rows.
constexpr int kFinalizeThreads = 256;
__global__ __launch_bounds__(kFinalizeThreads) void finalize_kernel(int64_t T, int K,
                                                                    const int32_t* __restrict__ slot,
                                                                    const int32_t* __restrict__ tile_base, int E,
                                                                    const int32_t* __restrict__ expert_offset,
                                                                    const int32_t* __restrict__ counts, int64_t cap,
                                                                    int32_t* __restrict__ dst_row,
                                                                    int32_t* __restrict__ recv_src_idx) {
    const int64_t nth = (int64_t)gridDim.x * kFinalizeThreads;
    for (int64_t i = (int64_t)blockIdx.x * kFinalizeThreads + threadIdx.x; i < T * K; i += nth) {
        const int64_t t = i / K;
        const int d = final_row(slot[i], t, tile_base, E, expert_offset, cap);
        dst_row[i] = d;
        if (d >= 0) recv_src_idx[d] = (int32_t)t;
    }
    fill_unused_grid<kFinalizeThreads>(recv_src_idx, expert_offset, counts, E, cap);
}

// Small batches (decode) and top-k above 8: one wave per (token, column chunk
// of U*64 16-byte vectors) stores its chunk to all K rows. Lanes 0..K-1 read
// the token's final rows and broadcast them; each lane loads its U vectors
// once and stores them to every destination row with non-temporal stores. A
// row is nvec 16-byte vectors of any payload (bf16 rows, or FP8 rows with
// their scales moved as the side payload by the chunk-0 wave).
template <int KM, int U>
__global__ __launch_bounds__(kScatterWaves* kWave) void scatter_bcast_kernel(const uint4* __restrict__ x, int64_t t0,
                                                                             int64_t T, int nvec, int nchunk, int K,
                                                                             const int32_t* __restrict__ dst_row,
                                                                             int64_t cap, uint4* __restrict__ recv_x,
                                                                             SideRows side) {
    const int lane = lane_id();
    const int64_t g = (int64_t)blockIdx.x * kScatterWaves + threadIdx.x / kWave;
    const int64_t tr = g / nchunk;
    const int64_t t = t0 + tr;
    if (t >= T) return;
    const int c = (int)(g - tr * nchunk);
    const int v0 = c * U * kWave;
    const uint4* xr = x + t * nvec;
    uint4 buf[U];  // loaded before the rows arrive
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int v = v0 + u * kWave + lane;
        if (v < nvec) buf[u] = xr[v];
    }
    int d = -1;
    if (lane < K) {
        const int p = dst_row[t * K + lane];
        d = (p >= 0 && p < cap) ? p : -1;
    }
    int dk[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        dk[k] = __builtin_amdgcn_readlane(d, k);
    }
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        if (dk[k] < 0) continue;
        uint4* dr = recv_x + (int64_t)dk[k] * nvec;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kWave + lane;
            if (v < nvec) store_nt(dr + v, buf[u]);
        }
        if (side.src && c == 0) copy_side_row(side, t, dk[k], lane);
    }
}

// Row copy to final rows, one wave per (token, U KB column chunk, group of S
// slots), WPB waves per block: the wave loads its chunk (U vectors of 16
// bytes per lane) and stores it to its S slots' receive rows with
// non-temporal stores. The waves of a chunk are adjacent (slot group
// fastest), so the chunk comes from HBM once and from L2 for the others.
// Measured on MI355X (prefill unless stated), with inputs that change every
// step, i.e. x in HBM: the waves of a chunk all wait for its one load, so
// fewer, fuller waves win: (S, U, WPB) = (2, 1, 16) takes 104 us against
// 131 us with one store per wave (S = 1) and 104-111 us with one wave
// storing all K rows; Zipf-skewed 184-186 against 246 us; at top-16 (32768
// tokens, hidden 4096) (2, 2, 4) takes 851 us against 868 for (2, 1, 16) and
// 910 for the broadcast kernel. With x in the Infinity Cache the shapes are
// within 3 %. Each wave needs its final rows after a single dependent load
// (dst_row, which the plan resolved), and stores nothing but its chunk:
// recording dst_row and recv_src_idx here, in the copy waves or in extra
// blocks, measured 3 us slower at prefill than in the plan. The grid covers
// tokens [t0, t_end). A row is nvec 16-byte vectors of any payload (bf16
// rows, or FP8 rows with their scales moved as the side payload by the
// chunk-0 waves).
template <int S, int U, int WPB>
__global__ __launch_bounds__(WPB* kWave) void scatter_kernel(const uint4* __restrict__ x, int64_t t0, int64_t t_end,
                                                            int nvec, int nchunk, int K,
                                                            const int32_t* __restrict__ dst_row, int64_t cap,
                                                            uint4* __restrict__ recv_x, SideRows side) {
    const int lane = lane_id();
    const unsigned wave = __builtin_amdgcn_readfirstlane((unsigned)(threadIdx.x / kWave));
    const unsigned g = blockIdx.x * (unsigned)WPB + wave;
    const int ng = (K + S - 1) / S;                 // slot groups per chunk
    const unsigned per = (unsigned)(nchunk * ng);  // waves per token
    const unsigned tt = g / per;
    const int64_t t = t0 + tt;
    if (t >= t_end) return;
    const int j = (int)(g - tt * per);
    const int c = j / ng;
    const int k0 = (j - c * ng) * S;
    uint4 buf[U];  // loads issued with the row load
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int v = (c * U + u) * kWave + lane;
        buf[u] = make_uint4(0, 0, 0, 0);
        if (v < nvec) buf[u] = x[t * nvec + v];
    }
    // lanes 0..K-1 load the token's rows (per-lane addresses keep the load on
    // the vector path); the wave keeps rows k0..k0+S-1
    int dl = -1;
    if (lane < K) {
        const int p = dst_row[t * K + lane];
        dl = (p >= 0 && p < cap) ? p : -1;
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int k = k0 + s;
        const int d = __builtin_amdgcn_readlane(dl, k < K ? k : 0);
        if (k >= K || d < 0) continue;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = (c * U + u) * kWave + lane;
            if (v < nvec) store_nt(recv_x + (int64_t)d * nvec + v, buf[u]);
        }
        if (side.src && c == 0) copy_side_row(side, t, d, lane);
    }
}

// Fused FP8 cast and dispatch apply (bf16 x in, e4m3fn rows and per-block
// scales out). One wave per (token, chunk of U*64 lanes): each lane holds
// CPL = 16 channels (two 16-byte bf16 vectors in, one 16-byte code vector
// out), so an 8-lane group holds one 128-channel block, whose absolute max
// comes from an 8-lane reduction (CPL = 8: 8-byte code vectors, 16-lane
// groups). The chunk is quantized once and its code vectors and block scales
// are stored to every destination row with non-temporal stores. Rows are H
// bytes; scales are [cap, H/128] (4 bytes, or 1 byte UE8M0). dst_row holds
// the plan's final rows. x is read with ordinary loads, which find it in the
// Infinity Cache when it is there (after a plan that pulled it in, or a
// producer that just wrote it); non-temporal loads went to HBM regardless.
// Prefill, fp32 scales, us: 59.7 against 62.2 with x rotating, 48.8 against
// 60.8 with x in the cache, 49.5 with no x loads at all (a probe), and 47.7
// for the code stores alone: the wave waits for its x chunk, not for its
// arithmetic or its scale stores (their removal: 62.0).
#ifndef CGD_CAST_CPL
#define CGD_CAST_CPL 16
#endif
constexpr int kCastCpl = CGD_CAST_CPL;  // channels per lane
template <int KM, int U, int FMT>
__global__ __launch_bounds__(kScatterWaves* kWave) void scatter_cast_kernel(
    const uint4* __restrict__ x, int64_t T, int nlv, int nchunk, int K, const int32_t* __restrict__ dst_row,
    int64_t cap, int64_t t0, void* __restrict__ recv_q, void* __restrict__ recv_s) {
    constexpr int kVin = kCastCpl / 8;             // 16-byte bf16 vectors per lane
    constexpr int kGroup = kFp8Block / kCastCpl;   // lanes per 128-channel block
    const int lane = lane_id();
    const int64_t g = (int64_t)blockIdx.x * kScatterWaves + threadIdx.x / kWave;
    const int64_t tr = g / nchunk;
    const int64_t t = t0 + tr;
    if (t >= T) return;
    const int c = (int)(g - tr * nchunk);
    const int v0 = c * U * kWave;  // first lane vector of the chunk (nlv per row)
    const int nsb = nlv / kGroup;
    const uint4* xr = x + t * (int64_t)nlv * kVin;
    uint4 buf[U][kVin];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int v = v0 + u * kWave + lane;
#pragma unroll
        for (int i = 0; i < kVin; ++i)
            if (v < nlv) buf[u][i] = xr[(int64_t)v * kVin + i];
    }
    int d = -1;
    if (lane < K) {
        const int p = dst_row[t * K + lane];
        d = (p >= 0 && p < cap) ? p : -1;
    }
    // quantize: a block never straddles two lane groups (nlv % kGroup == 0)
    Fp8Scale sc[U];
    uint4 code16[U];
    uint2 code8[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int v = v0 + u * kWave + lane;
        float m = 0.0f;
        if (v < nlv) {
#pragma unroll
            for (int i = 0; i < kVin; ++i) m = fmaxf(m, absmax_bf16x8(buf[u][i]));
        }
        m = (kGroup == 8) ? group8_max(m) : group16_max(m);
        sc[u] = fp8_block_scale(m, FMT);
        if (kCastCpl == 16)
            code16[u] = quantize_bf16x16(buf[u][0], buf[u][kVin - 1], sc[u].mul);
        else
            code8[u] = quantize_bf16x8(buf[u][0], sc[u].mul);
    }
    int dk[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) dk[k] = __builtin_amdgcn_readlane(d, k);
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        if (dk[k] < 0) continue;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kWave + lane;
            if (v >= nlv) continue;
            if (kCastCpl == 16)
                store_nt(static_cast<uint4*>(recv_q) + (int64_t)dk[k] * nlv + v, code16[u]);
            else
                store_nt(static_cast<uint2*>(recv_q) + (int64_t)dk[k] * nlv + v, code8[u]);
            if ((lane & (kGroup - 1)) == 0) {
                const int64_t si = (int64_t)dk[k] * nsb + v / kGroup;
                if (FMT == 2)
                    static_cast<uint8_t*>(recv_s)[si] = (uint8_t)sc[u].ue8m0;
                else
                    static_cast<float*>(recv_s)[si] = sc[u].scale;
            }
        }
    }
}

hipError_t preload_dispatch() {
    hipFuncAttributes a;
    return hipFuncGetAttributes(&a, reinterpret_cast<const void*>(&finalize_kernel));
}

// Dispatch workspace: ticket | tile bases int32 [tiles, E] | packed slot
// words int32 [T, K] (rank_kernel -> finalize_kernel) | per-expert slot
// counts int32 [E] | segment offsets int32 [E+1] of the packed layout (its
// own copy, so the packed entry points need no offsets argument).
struct DispatchWs {
    unsigned int* ticket;
    int32_t* tile_base;
    int32_t* slot_pack;
    int32_t* counts;
    int32_t* packed_offset;
    int32_t* rank_part;  // per-tile distinct tokens per rank (fused layout), [tiles, R]; last, so the
                         // offsets of the other arrays do not depend on R
};

static size_t rnd256(size_t b) { return (b + 255) / 256 * 256; }

static size_t tile_bytes(int64_t T, int E) {
    const int64_t ntiles = T <= 0 ? 1 : (T + kRankTile - 1) / kRankTile;
    return rnd256((size_t)ntiles * (size_t)E * sizeof(int32_t));
}

static size_t slot_bytes(int64_t T, int K) { return rnd256((size_t)(T > 0 ? T : 0) * (size_t)K * sizeof(int32_t)); }

size_t dispatch_workspace_bytes(int64_t T, int K, int E, int R) {
    return kTicketBytes + tile_bytes(T, E) + slot_bytes(T, K) + rnd256((size_t)E * 4) + rnd256((size_t)(E + 1) * 4) +
           tile_bytes(T, R);
}

static DispatchWs dispatch_ws(const void* workspace, int64_t T, int K, int E) {
    char* p = static_cast<char*>(const_cast<void*>(workspace));
    DispatchWs w;
    w.ticket = reinterpret_cast<unsigned int*>(p);
    p += kTicketBytes;
    w.tile_base = reinterpret_cast<int32_t*>(p);
    p += tile_bytes(T, E);
    w.slot_pack = reinterpret_cast<int32_t*>(p);
    p += slot_bytes(T, K);
    w.counts = reinterpret_cast<int32_t*>(p);
    p += rnd256((size_t)E * 4);
    w.packed_offset = reinterpret_cast<int32_t*>(p);
    p += rnd256((size_t)(E + 1) * 4);
    w.rank_part = reinterpret_cast<int32_t*>(p);
    return w;
}

// Batches with fewer slots (decode) use the broadcast kernel: one wave per
// (token, chunk) stores its chunk to all K rows, so a small grid still
// moves whole rows per wave.
constexpr int64_t kRowCopyMinSlots = 16384;
constexpr int kRowCopyMaxTopk = 8;  // above: 2 KB chunks, 4 waves per block
#ifndef CGD_ROW_SLOTS
#define CGD_ROW_SLOTS 2
#endif
constexpr int kRowSlots = CGD_ROW_SLOTS;  // slots per wave of the row copy

// The row copy that follows a plan launch which pulled x toward the caches
// (the non-cached dispatch) runs fewer waves per CU: x then arrives from the
// Infinity Cache, so fewer stores in flight keep up, and HBM sees fewer
// concurrent destination streams. Blocks of CGD_ROW_COPY_PF_WAVES waves with
// an LDS reservation of CGD_ROW_COPY_PF_LDS bytes each (5 blocks of 4 waves
// per CU), CGD_ROW_COPY_PF_LDS_WIDE above top-8 (6 blocks of 4). Whole
// dispatch (plan + rows), inputs rotating, us: prefill 103.3 against 107.6
// with the cached copy's 2 blocks of 16 waves, Zipf-skewed 191.2 against
// 199.2, top-16 888 against 897. The cached copy (x from HBM) keeps its
// shape: there the same change costs 120 against 98.7 us at prefill.
#ifndef CGD_ROW_COPY_PF_WAVES
#define CGD_ROW_COPY_PF_WAVES 4
#endif
#ifndef CGD_ROW_COPY_PF_LDS
#define CGD_ROW_COPY_PF_LDS 32768
#endif
#ifndef CGD_ROW_COPY_PF_LDS_WIDE
#define CGD_ROW_COPY_PF_LDS_WIDE 27000
#endif

template <int S, int U, int WPB>
static void launch_row_copy(int64_t T, int K, hipStream_t s, const void* x, int nvec, const int32_t* dst_row,
                            int64_t cap, void* recv_x, const SideRows& side, size_t lds = 0) {
    const int nchunk = (nvec + U * kWave - 1) / (U * kWave);
    const int64_t per = (int64_t)nchunk * ((K + S - 1) / S);  // waves per token
    const int64_t tper = tokens_per_launch(per);
    for (int64_t t0 = 0; t0 < T; t0 += tper) {
        const int64_t nt = std::min<int64_t>(tper, T - t0);
        const int64_t blocks = (nt * per + WPB - 1) / WPB;
        hipLaunchKernelGGL((scatter_kernel<S, U, WPB>), dim3((unsigned)blocks), dim3(WPB * kWave), lds, s,
                           reinterpret_cast<const uint4*>(x), t0, t0 + nt, nvec, nchunk, K, dst_row, cap,
                           reinterpret_cast<uint4*>(recv_x), side);
    }
}

template <int U>
static void launch_bcast_u(int64_t T, int K, hipStream_t s, const void* x, int nvec, const int32_t* dst_row,
                           int64_t cap, void* recv_x, const SideRows& side) {
    const int nchunk = (nvec + U * kWave - 1) / (U * kWave);
    const int64_t tper = tokens_per_launch(nchunk);
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    uint4* rv = reinterpret_cast<uint4*>(recv_x);
    const dim3 block(kScatterWaves * kWave);
    for (int64_t t0 = 0; t0 < T; t0 += tper) {
        const int64_t nt = std::min<int64_t>(tper, T - t0);
        const dim3 grid((unsigned)((nt * nchunk + kScatterWaves - 1) / kScatterWaves));
#define CGD_SCATTER(KM)                                                                                            \
    hipLaunchKernelGGL((scatter_bcast_kernel<KM, U>), grid, block, 0, s, xv, t0, t0 + nt, nvec, nchunk, K, dst_row, \
                       cap, rv, side)
        if (K <= 2)
            CGD_SCATTER(2);
        else if (K <= 4)
            CGD_SCATTER(4);
        else if (K <= 8)
            CGD_SCATTER(8);
        else
            CGD_SCATTER(16);
#undef CGD_SCATTER
    }
}

// Rows moved to the final rows of a handle (the apply of a plan, cached
// dispatch, the packed dispatch): the row copy for larger batches (2 KB
// chunks in blocks of 4 waves above top-8), the broadcast kernel for small
// ones. after_plan: the copy follows a plan launch that prefetched x.
static void launch_scatter(int64_t T, int K, hipStream_t s, const void* x, int nvec, const int32_t* dst_row,
                           int64_t cap, void* recv_x, const SideRows& side, bool after_plan = false) {
    if (T <= 0) return;
    if (T * K < kRowCopyMinSlots)
        launch_bcast_u<1>(T, K, s, x, nvec, dst_row, cap, recv_x, side);
    else if (K > kRowCopyMaxTopk)
        launch_row_copy<kRowSlots, 2, 4>(T, K, s, x, nvec, dst_row, cap, recv_x, side,
                                         after_plan ? CGD_ROW_COPY_PF_LDS_WIDE : 0);
    else if (after_plan)
        launch_row_copy<kRowSlots, 1, CGD_ROW_COPY_PF_WAVES>(T, K, s, x, nvec, dst_row, cap, recv_x, side,
                                                              CGD_ROW_COPY_PF_LDS);
    else
        launch_row_copy<kRowSlots, 1, kSlotWaves>(T, K, s, x, nvec, dst_row, cap, recv_x, side);
}

static SideRows no_side() { return SideRows{nullptr, 0, 0, 0, 0, nullptr}; }

static SideRows fp8_side(const void* scales, int64_t st, int64_t sb, int H, int fmt, void* recv_scales) {
    return SideRows{scales, st, sb, H / kFp8Block, fmt == 2 ? 1 : 4, recv_scales};
}

// Compute units of the current device (cached per device; host threads may
// race on the cache, each storing the same value).
int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// The plan, from the routing alone: rank_kernel, which completes the handle
// (dst_row, recv_src_idx with its -1 fill) of a one-tile batch itself, else
// finalize_kernel after it. A one-tile batch with many spare rows (a large
// fixed capacity or alignment) takes the FUSED form without rows to move:
// every block plans the tile in LDS and fills a share of the spare rows.
// px (optional, pbytes of x): a plan of several tiles followed by a row copy
// of x adds kPrefetchBlocks blocks that pull x toward the caches meanwhile.
constexpr int64_t kSpareRowsPerBlock = 2048;
static hipError_t launch_rank(const int64_t* topk_idx, int64_t T, int K, int E, int A, int seg_cap, int64_t cap,
                              int32_t* expert_offset, int32_t* nrecv, int32_t* dst_row, int32_t* recv_src_idx,
                              int32_t* packed_count, int32_t* stats, const DispatchWs& w, hipStream_t stream,
                              const LayoutOut* layout = nullptr, const void* px = nullptr, int64_t pbytes = 0) {
    int ebits = 0;
    while ((1 << ebits) < E) ++ebits;
    const int ntiles = (int)(T <= 0 ? 1 : (T + kRankTile - 1) / kRankTile);
    const dim3 block(kRankTile);
    const size_t lds = rank_lds_bytes(E, K);
    const TileOut to{dst_row, recv_src_idx, cap, nullptr, 0, 1, nullptr, -1, 0, nullptr, nullptr};  // no rows to move
    const LayoutOut none{1, 1, nullptr, nullptr, nullptr, nullptr};
    const LayoutOut& lo = layout ? *layout : none;
    const int64_t spare = cap - std::min<int64_t>(cap, std::max<int64_t>(T, 0) * K);
    const int64_t fill_blocks = std::min<int64_t>(spare / kSpareRowsPerBlock, device_cus());
    const uint4* pv = reinterpret_cast<const uint4*>(px);
    const int64_t pvecs = px ? pbytes / 16 : 0;
#define CGD_RANK(RW, LAYOUT, FUSED, GRID, PV, PN)                                                                       \
    hipLaunchKernelGGL((rank_kernel<RW, LAYOUT, FUSED>), GRID, block, lds, stream, topk_idx, T, K, E, ebits, A, seg_cap, \
                       w.slot_pack, w.tile_base, expert_offset, nrecv, w.counts, packed_count, stats, w.ticket, lo, to,  \
                       ntiles, PV, PN)
    if (ntiles == 1 && fill_blocks > 1) {
        const dim3 fgrid((unsigned)fill_blocks);
        if (!layout)
            CGD_RANK(1, false, true, fgrid, nullptr, 0);
        else if (layout->R <= 64)
            CGD_RANK(1, true, true, fgrid, nullptr, 0);
        else
            CGD_RANK(6, true, true, fgrid, nullptr, 0);
        return hipGetLastError();
    }
    const int extra = (ntiles > 1 && pvecs > 0) ? kPrefetchBlocks : 0;
    const dim3 grid(ntiles + extra);
    if (!layout)
        CGD_RANK(1, false, false, grid, pv, pvecs);
    else if (layout->R <= 64)
        CGD_RANK(1, true, false, grid, pv, pvecs);
    else
        CGD_RANK(6, true, false, grid, pv, pvecs);
#undef CGD_RANK
    if (ntiles > 1) {
        // a thread per slot (grid capped, the kernel strides), and at least
        // kFillThreads threads for the fill
        const int64_t n = T * K;
        const int64_t blocks = std::max<int64_t>(std::min<int64_t>((n + kFinalizeThreads - 1) / kFinalizeThreads, 65536),
                                                 kFillThreads / kFinalizeThreads);
        hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)blocks), dim3(kFinalizeThreads), 0, stream, T, K,
                           w.slot_pack, w.tile_base, E, expert_offset, w.counts, cap, dst_row, recv_src_idx);
    }
    return hipGetLastError();
}

hipError_t launch_layout_and_plan(const int64_t* topk_idx, int64_t T, int K, int E, int R, int A, int64_t cap,
                                  int32_t* ntpr, int32_t* ntpe, uint8_t* itr, int32_t* expert_offset, int32_t* nrecv,
                                  int32_t* recv_src_idx, int32_t* dst_row, void* workspace, hipStream_t stream,
                                  const void* x, int64_t x_bytes) {
    const DispatchWs w = dispatch_ws(workspace, T, K, E);
    const LayoutOut lo{R, E / R, ntpr, ntpe, itr, w.rank_part};
    return launch_rank(topk_idx, T, K, E, A, -1, cap, expert_offset, nrecv, dst_row, recv_src_idx, nullptr, nullptr, w,
                       stream, &lo, x, x_bytes);
}

hipError_t launch_dispatch_plan(const int64_t* topk_idx, int64_t T, int K, int E, int A, int64_t cap,
                                int32_t* expert_offset, int32_t* nrecv, int32_t* recv_src_idx, int32_t* dst_row,
                                void* workspace, hipStream_t stream, const void* x, int64_t x_bytes) {
    return launch_rank(topk_idx, T, K, E, A, -1, cap, expert_offset, nrecv, dst_row, recv_src_idx, nullptr, nullptr,
                       dispatch_ws(workspace, T, K, E), stream, nullptr, x, x_bytes);
}

// Residency of the cast on dispatch: an LDS reservation of this many bytes
// per 4-wave block leaves 6 blocks per CU. Prefill, fp32 scales, inputs
// rotating: 61.2 us against 62.6-62.7 with 8 blocks (no reservation); 5
// blocks 62.6, 4 blocks 62.6, 3 blocks 63.8.
#ifndef CGD_SCATTER_CAST_LDS
#define CGD_SCATTER_CAST_LDS 27000
#endif
template <int U, int FMT>
static void launch_scatter_cast_u(const void* x, int64_t T, int H, int K, const int32_t* dst_row, int64_t cap,
                                  void* recv_q, void* recv_s, hipStream_t s) {
    const int nlv = H / kCastCpl;
    const int nchunk = (nlv + U * kWave - 1) / (U * kWave);
    const int64_t tper = tokens_per_launch(nchunk);
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    const dim3 block(kScatterWaves * kWave);
    for (int64_t t0 = 0; t0 < T; t0 += tper) {
        const int64_t nt = std::min<int64_t>(tper, T - t0);
        const dim3 grid((unsigned)((nt * nchunk + kScatterWaves - 1) / kScatterWaves));
#define CGD_SCATTER_CAST(KM)                                                                                        \
    hipLaunchKernelGGL((scatter_cast_kernel<KM, U, FMT>), grid, block, CGD_SCATTER_CAST_LDS, s, xv, t0 + nt, nlv,  \
                       nchunk, K, dst_row, cap, t0, recv_q, recv_s)
        if (K <= 2)
            CGD_SCATTER_CAST(2);
        else if (K <= 4)
            CGD_SCATTER_CAST(4);
        else if (K <= 8)
            CGD_SCATTER_CAST(8);
        else
            CGD_SCATTER_CAST(16);
#undef CGD_SCATTER_CAST
    }
}

// Chunks of U vectors per lane unless that leaves fewer than kMinScatterWaves
// waves, as for a decode batch: then 1 vector per lane.
constexpr int64_t kMinScatterWaves = 4096;

#ifndef CGD_SCATTER_CAST_U
#define CGD_SCATTER_CAST_U 2
#endif

static void launch_scatter_cast(const void* x, int64_t T, int H, int K, int fmt, const int32_t* dst_row,
                                int64_t cap, void* recv_q, void* recv_s, hipStream_t s) {
    if (T <= 0) return;
    constexpr int U = CGD_SCATTER_CAST_U;
    const bool wide = T * ((H / kCastCpl + U * kWave - 1) / (U * kWave)) >= kMinScatterWaves;
#define CGD_CAST(FMT)                                                                 \
    do {                                                                              \
        if (wide)                                                                     \
            launch_scatter_cast_u<U, FMT>(x, T, H, K, dst_row, cap, recv_q, recv_s, s); \
        else                                                                          \
            launch_scatter_cast_u<1, FMT>(x, T, H, K, dst_row, cap, recv_q, recv_s, s); \
    } while (0)
    if (fmt == 0)
        CGD_CAST(0);
    else if (fmt == 1)
        CGD_CAST(1);
    else
        CGD_CAST(2);
#undef CGD_CAST
}

hipError_t launch_dispatch_cached_cast_fp8(const void* x, int64_t T, int H, int K, int fmt, const int32_t* dst_row,
                                           void* recv_q, void* recv_s, int64_t cap, hipStream_t stream) {
    if (T <= 0) return hipSuccess;  // nothing to enqueue
    launch_scatter_cast(x, T, H, K, fmt, dst_row, cap, recv_q, recv_s, stream);
    return hipGetLastError();
}

// Plan and bf16 apply of a batch of at most one tile in one launch (the FUSED
// rank kernel); seg_cap >= 0 for the fixed-capacity packed layout; with
// layout, get_dispatch_layout's outputs from the same launch; fmt >= 0: the
// rows receive x cast to FP8 (codes in recv_x, scales in recv_s).
static hipError_t launch_fused(const int64_t* topk_idx, int64_t T, int K, int E, int A, int seg_cap, const void* x,
                               int H, void* recv_x, int64_t cap, int32_t* expert_offset, int32_t* nrecv,
                               int32_t* recv_src_idx,
                               int32_t* dst_row, int32_t* packed_count, int32_t* stats, const DispatchWs& w,
                               hipStream_t stream, const LayoutOut* layout = nullptr, int fmt = -1,
                               void* recv_s = nullptr) {
    int ebits = 0;
    while ((1 << ebits) < E) ++ebits;
    const int nvec = H / 8;
    const int nchunk = (nvec + kWave - 1) / kWave;
    // one block per CU where that leaves at most kFusedItems items per wave:
    // every block plans the whole batch in LDS, so blocks sharing a CU would
    // share its LDS bandwidth for that
    const int64_t items = T * nchunk;
    const int64_t per_block = (int64_t)kRankWaves * kFusedItems;
    int64_t blocks = std::max<int64_t>(std::min<int64_t>((items + kRankWaves - 1) / kRankWaves, device_cus()),
                                       (items + per_block - 1) / per_block);
    // in a grid of several blocks the first block (the first two with the
    // layout outputs, in a grid of three or more) moves no rows: the others
    // hold every item
    const int64_t need = (items + per_block - 1) / per_block;
    if (blocks > 1) blocks = std::max<int64_t>(blocks, 1 + need);
    if (blocks > 2 && layout) blocks = std::max<int64_t>(blocks, 2 + need);
    const dim3 grid((unsigned)std::max<int64_t>(1, blocks)), block(kRankTile);
    const LayoutOut none{1, 1, nullptr, nullptr, nullptr, nullptr};
    const bool cast = fmt >= 0;
    const TileOut fc{dst_row, recv_src_idx, cap, reinterpret_cast<const uint4*>(x), nvec, nchunk,
                     cast ? nullptr : reinterpret_cast<uint4*>(recv_x), fmt, H / kFp8Block,
                     cast ? reinterpret_cast<uint2*>(recv_x) : nullptr, cast ? recv_s : nullptr};
    const size_t lds = rank_lds_bytes(E, K);
#define CGD_FUSED(RW, LAYOUT, CAST, LO)                                                                       \
    hipLaunchKernelGGL((rank_kernel<RW, LAYOUT, true, CAST>), grid, block, lds, stream, topk_idx, T, K, E, ebits, A, \
                       seg_cap, w.slot_pack, w.tile_base, expert_offset, nrecv, w.counts, packed_count, stats,       \
                       w.ticket, LO, fc, 1, nullptr, 0)
    if (!layout) {
        if (cast)
            CGD_FUSED(1, false, true, none);
        else
            CGD_FUSED(1, false, false, none);
    } else if (layout->R <= 64) {
        if (cast)
            CGD_FUSED(1, true, true, *layout);
        else
            CGD_FUSED(1, true, false, *layout);
    } else {
        if (cast)
            CGD_FUSED(6, true, true, *layout);
        else
            CGD_FUSED(6, true, false, *layout);
    }
#undef CGD_FUSED
    return hipGetLastError();
}

// The non-cached cast on dispatch: the plan (with the layout outputs when
// `layout` is given), whose spare blocks pull x into the caches while it
// runs when x fits there, then the cast to its rows, which then reads x from
// there (top-16 stress, 268 MB of x: 561 us with the prefetch against 520
// for the plan and the cast as two calls).
static hipError_t launch_plan_and_cast(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E, int A,
                                       int fmt, void* recv_q, void* recv_s, int64_t cap, int32_t* expert_offset,
                                       int32_t* nrecv, int32_t* recv_src_idx, int32_t* dst_row, const DispatchWs& w,
                                       hipStream_t stream, const LayoutOut* layout) {
    if (T > 0 && dispatch_fuses(T))  // one tile (decode): plan, cast and rows in one launch
        return launch_fused(topk_idx, T, K, E, A, -1, x, H, recv_q, cap, expert_offset, nrecv, recv_src_idx, dst_row,
                            nullptr, nullptr, w, stream, layout, fmt, recv_s);
    const int64_t xb = T * (int64_t)H * 2;
    hipError_t err = launch_rank(topk_idx, T, K, E, A, -1, cap, expert_offset, nrecv, dst_row, recv_src_idx, nullptr,
                                 nullptr, w, stream, layout, xb <= kPrefetchMaxBytes ? x : nullptr, xb);
    if (err != hipSuccess) return err;
    if (T > 0) launch_scatter_cast(x, T, H, K, fmt, dst_row, cap, recv_q, recv_s, stream);
    return hipGetLastError();
}

hipError_t launch_dispatch_cast_fp8(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E, int A,
                                    int fmt, void* recv_q, void* recv_s, int64_t cap, int32_t* expert_offset,
                                    int32_t* nrecv, int32_t* recv_src_idx, int32_t* dst_row, void* workspace,
                                    hipStream_t stream) {
    return launch_plan_and_cast(x, T, H, topk_idx, K, E, A, fmt, recv_q, recv_s, cap, expert_offset, nrecv,
                                recv_src_idx, dst_row, dispatch_ws(workspace, T, K, E), stream, nullptr);
}

hipError_t launch_layout_and_dispatch_cast_fp8(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E,
                                               int R, int A, int fmt, void* recv_q, void* recv_s, int64_t cap,
                                               int32_t* ntpr, int32_t* ntpe, uint8_t* itr, int32_t* expert_offset,
                                               int32_t* nrecv, int32_t* recv_src_idx, int32_t* dst_row,
                                               void* workspace, hipStream_t stream) {
    const DispatchWs w = dispatch_ws(workspace, T, K, E);
    const LayoutOut lo{R, E / R, ntpr, ntpe, itr, w.rank_part};
    return launch_plan_and_cast(x, T, H, topk_idx, K, E, A, fmt, recv_q, recv_s, cap, expert_offset, nrecv,
                                recv_src_idx, dst_row, w, stream, &lo);
}

bool dispatch_fuses(int64_t T) { return T <= kRankTile; }

hipError_t launch_dispatch_fused(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E, int A,
                                 void* recv_x, int64_t cap, int32_t* expert_offset, int32_t* nrecv,
                                 int32_t* recv_src_idx, int32_t* dst_row, void* workspace, hipStream_t stream) {
    return launch_fused(topk_idx, T, K, E, A, -1, x, H, recv_x, cap, expert_offset, nrecv, recv_src_idx, dst_row,
                        nullptr, nullptr, dispatch_ws(workspace, T, K, E), stream);
}

hipError_t launch_layout_and_dispatch_fused(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E,
                                            int R, int A, void* recv_x, int64_t cap, int32_t* ntpr, int32_t* ntpe,
                                            uint8_t* itr, int32_t* expert_offset, int32_t* nrecv,
                                            int32_t* recv_src_idx, int32_t* dst_row, void* workspace,
                                            hipStream_t stream) {
    const DispatchWs w = dispatch_ws(workspace, T, K, E);
    const LayoutOut lo{R, E / R, ntpr, ntpe, itr, w.rank_part};
    return launch_fused(topk_idx, T, K, E, A, -1, x, H, recv_x, cap, expert_offset, nrecv, recv_src_idx, dst_row,
                        nullptr, nullptr, w, stream, &lo);
}

static hipError_t packed_launches(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E,
                                  int expert_capacity, int fmt, void* recv_x, void* recv_s, int32_t* packed_count,
                                  int32_t* recv_src_info, int32_t* dst_row, int32_t* stats, const DispatchWs& w,
                                  hipStream_t stream, const LayoutOut* layout) {
    const int64_t cap = (int64_t)E * expert_capacity;
    if (dispatch_fuses(T) && (fmt < 0 || T > 0))  // one tile: plan (cast) and rows in one launch
        return launch_fused(topk_idx, T, K, E, 1, expert_capacity, x, H, recv_x, cap, w.packed_offset, nullptr,
                            recv_src_info, dst_row, packed_count, stats, w, stream, layout, fmt, recv_s);
    // the bf16 row copy after the plan wants x in the caches at any size; the
    // cast only while x stays there (kPrefetchMaxBytes)
    const int64_t xb = T * (int64_t)H * 2;
    const void* px = (fmt < 0 || xb <= kPrefetchMaxBytes) ? x : nullptr;
    hipError_t err = launch_rank(topk_idx, T, K, E, 1, expert_capacity, cap, w.packed_offset, nullptr, dst_row,
                                 recv_src_info, packed_count, stats, w, stream, layout, px, xb);
    if (err != hipSuccess) return err;
    if (fmt < 0)
        launch_scatter(T, K, stream, x, H / 8, dst_row, cap, recv_x, no_side(), true);
    else
        launch_scatter_cast(x, T, H, K, fmt, dst_row, cap, recv_x, recv_s, stream);
    return hipGetLastError();
}

hipError_t launch_dispatch_packed(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E,
                                  int expert_capacity, int fmt, void* recv_x, void* recv_s, int32_t* packed_count,
                                  int32_t* recv_src_info, int32_t* dst_row, int32_t* stats, void* workspace,
                                  hipStream_t stream) {
    return packed_launches(x, T, H, topk_idx, K, E, expert_capacity, fmt, recv_x, recv_s, packed_count,
                           recv_src_info, dst_row, stats, dispatch_ws(workspace, T, K, E), stream, nullptr);
}

hipError_t launch_layout_and_dispatch_packed(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E,
                                             int R, int expert_capacity, int fmt, void* recv_x, void* recv_s,
                                             int32_t* packed_count, int32_t* recv_src_info, int32_t* dst_row,
                                             int32_t* stats, int32_t* ntpr, int32_t* ntpe, uint8_t* itr,
                                             void* workspace, hipStream_t stream) {
    const DispatchWs w = dispatch_ws(workspace, T, K, E);
    const LayoutOut lo{R, E / R, ntpr, ntpe, itr, w.rank_part};
    return packed_launches(x, T, H, topk_idx, K, E, expert_capacity, fmt, recv_x, recv_s, packed_count,
                           recv_src_info, dst_row, stats, w, stream, &lo);
}

hipError_t launch_dispatch_cached(const void* x, int64_t T, int H, int K, const int32_t* dst_row, void* recv_x,
                                  int64_t cap, hipStream_t stream, bool after_plan) {
    if (T <= 0) return hipSuccess;  // nothing to enqueue
    launch_scatter(T, K, stream, x, H / 8, dst_row, cap, recv_x, no_side(), after_plan);
    return hipGetLastError();
}

hipError_t launch_dispatch_cached_fp8(const void* xq, const void* xs, int64_t st, int64_t sb, int fmt, int64_t T,
                                      int H, int K, const int32_t* dst_row, void* recv_q, void* recv_s, int64_t cap,
                                      hipStream_t stream) {
    if (T <= 0) return hipSuccess;  // nothing to enqueue
    launch_scatter(T, K, stream, xq, H / 16, dst_row, cap, recv_q, fp8_side(xs, st, sb, H, fmt, recv_s));
    return hipGetLastError();
}

}  // namespace cgd
