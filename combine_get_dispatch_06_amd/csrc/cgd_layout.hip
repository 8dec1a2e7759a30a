// get_dispatch_layout on gfx950.
//
// Computes, from topk_idx [T,K] (get_dispatch_layout API page, "Return
// Values"): per-expert slot counts, per-rank distinct-token counts and the
// is_token_in_rank matrix. Rank r owns experts [r*L, (r+1)*L) (DeepEP legacy
// test analysis page, low-latency per-expert check).
//
// One launch. Each block takes a tile of tokens, one per thread:
//   1. the tile's topk_idx is staged in LDS with coalesced loads;
//   2. each thread adds its slots to an LDS expert histogram and builds the
//      bitmask of ranks its token touches;
//   3. distinct tokens per rank: per wave, one ballot per rank and a popcount
//      of the lanes whose token holds it;
//   4. the tile's is_token_in_rank rows (a contiguous byte range) are written
//      with 16-byte stores;
//   5. the tiles' counts are combined across blocks without pre-zeroed
//      outputs or a second launch: get_dispatch_layout alone
//      (layout_acc_kernel, 512-token tiles) adds them to counted 64-bit
//      accumulators, and the block that adds last to a word writes it; the
//      rank-granular plan form (layout_kernel, 256-token tiles, which also
//      needs per-tile prefixes) publishes per-block partials that the last
//      block to finish sums.
// The NPU implementation on the API page ("Internal Logic", "Multi-Core
// Strategy") also splits tokens over cores and aggregates partial results
// across cores.
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

// The per-token FP8 cast that CAST blocks write (codes [T, H], row-major
// scales [T, H/128]).
struct CastOut {
    int H, fmt;
    uint4* q;
    void* scales;
};

// Blocks past the first nblk (the tiles) take no part in the plan: they pull
// px (pvecs 16-byte vectors, the x of the rank-granular apply that follows)
// toward the caches, or with CAST cast px (bf16 [T, H]) to FP8 for the apply.
template <int RW, bool NPLAN = false, bool CAST = false>  // RW: 64-bit words of the rank mask: 1 (R <= 64) or 6 (R <= 384)
__global__ __launch_bounds__(kLayoutTile) void layout_kernel(const int64_t* __restrict__ topk_idx, int64_t T, int K,
                                                             int E, int R, int L, int32_t* __restrict__ ntpr,
                                                             int32_t* __restrict__ ntpe, uint8_t* __restrict__ itr,
                                                             int32_t* __restrict__ partial,
                                                             unsigned int* __restrict__ ticket, NormalPlanOut np,
                                                             int nblk, const uint4* __restrict__ px, int64_t pvecs,
                                                             CastOut co) {
    if ((int)blockIdx.x >= nblk) {
        if (CAST)
            cast_rows<kLayoutTile>(px, T, co.H, co.fmt, co.q, co.scales, (int)blockIdx.x - nblk,
                                   (int)gridDim.x - nblk);
        else
            prefetch_rows<kLayoutTile>(px, pvecs, (int)blockIdx.x - nblk, (int)gridDim.x - nblk);
        return;
    }
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

    // top-k <= kDirectTopk: the token's routing straight into registers
    // (as the layout alone below); larger top-k: the coalesced stage
    const bool direct = K <= kDirectTopk;
    int64_t raw[kMaxTopk];
    {
        const int64_t* tok = topk_idx + (t0 + min(tid, max(nt - 1, 0))) * K;
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k) raw[k] = (direct && tid < nt && k < K) ? tok[k] : -1;
    }
    for (int i = tid; i < E; i += kLayoutTile) {
        s_hist[i] = 0;
        s_rank_of[i] = (int16_t)(i / L);
    }
    for (int i = tid; i < R; i += kLayoutTile) s_rank[i] = 0;
    if (!direct) stage_routing<kMaxTopk, kLayoutTile>(topk_idx + t0 * K, nt * K, E, s_idx);
    __syncthreads();

    int e[kMaxTopk];
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
        if (direct)
            e[k] = (raw[k] >= 0 && raw[k] < E) ? (int)raw[k] : -1;
        else
            e[k] = (tid < nt && k < K) ? s_idx[tid * K + k] : -1;
    }
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

    if (nblk == 1) {
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
    if (!last_block_done(ticket, nblk)) return;

    // each thread sums columns tid and tid + 256 (W <= 512 + 384): the loads
    // of both, 16 blocks at a time, are in flight together, so a column count
    // just above the block size costs no second round trip
    for (int i0 = tid; i0 < W; i0 += 2 * kLayoutTile) {
        const int i1 = i0 + kLayoutTile;
        int s0 = 0, s1 = 0;
        for (int b0 = 0; b0 < nblk; b0 += 16) {
            int v0[16], v1[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                v0[j] = (b0 + j < nblk) ? partial[(int64_t)(b0 + j) * W + i0] : 0;
                v1[j] = (b0 + j < nblk && i1 < W) ? partial[(int64_t)(b0 + j) * W + i1] : 0;
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                s0 += v0[j];
                s1 += v1[j];
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = h ? i1 : i0;
            const int s = h ? s1 : s0;
            if (i >= W) continue;
            if (i < E) {
                ntpe[i] = s;
                if (NPLAN && np.nrecv) np.nrecv[i] = (s + np.A - 1) / np.A * np.A;
            } else {
                ntpr[i - E] = s;
                if (NPLAN) s_rank[i - E] = s;
            }
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

// Rows of the one-launch rank-granular dispatch (normal_fused_kernel).
struct NormalRowsOut {
    const uint4* x;  // bf16 [T, H] as nvec 16-byte vectors per token
    int nvec, nchunk;
    const float* topk_w;  // read only with recv_topk_idx
    uint4* recv_x;
    int64_t cap;
    int32_t* send_row;
    int32_t* recv_src_idx;
    int64_t* recv_topk_idx;  // nullptr: no top-k metadata
    float* recv_topk_w;
    // CAST form: the per-token FP8 cast of x (codes [T, H] as nvec 8-byte
    // vectors per token, row-major scales [T, nsb], fp32 or one UE8M0 byte
    // for fmt 2), and the receive rows of codes and scales in place of recv_x
    int fmt, nsb;
    uint2* xq;
    void* xs;
    uint2* rq;
    void* rs;
};
constexpr int kNormalFusedItems = 4;  // (token, 1 KB chunk) items per wave at most

// A batch of at most one tile (decode), rank-granular, in one launch: the
// layout, the plan and the rows. Every block plans the whole tile in LDS (the
// same tile work as layout_kernel: rank masks, per-wave ballots per rank as
// group words, per-rank distinct-token counts, and a block scan of those
// counts into the rank offsets), which costs less than a second launch. In a
// grid of several blocks, block 0 alone writes the layout and plan outputs
// (the workspace's plan included, so that a later apply can read it) and
// moves no rows; the waves of the other blocks each take up to
// kNormalFusedItems (token, chunk) items. A token's row on rank r is the rank
// offset + the rank's tokens in earlier waves + the popcount of the group word
// below the token, as the two-launch path computes it from the workspace.
// Each item's x chunk is loaded once (after the routing is staged: loads
// complete in issue order) and stored to every row of the token with
// non-temporal stores; a token's chunk-0 item writes its send_row entries,
// recv_src_idx and each row's rank-local top-k ids and weights. Every block
// fills a share of the rows past the data. CAST: each item also casts its
// chunk to FP8 as the per-token cast does (a 16-lane group holds one
// 128-channel block), writes the codes and scales to the cast tuple, and
// moves them, not the bf16 chunk, to the token's rows.
template <int RW, bool CAST>
__global__ __launch_bounds__(kLayoutTile) void normal_fused_kernel(const int64_t* __restrict__ topk_idx, int64_t T,
                                                                   int K, int E, int R, int L,
                                                                   int32_t* __restrict__ ntpr,
                                                                   int32_t* __restrict__ ntpe,
                                                                   uint8_t* __restrict__ itr, NormalPlanOut np,
                                                                   NormalRowsOut ro) {
    constexpr int kGroups = kLayoutTile / kWave;
    __shared__ int32_t s_idx[kLayoutTile * kMaxTopk];
    __shared__ uint64_t s_mask[kLayoutTile * RW];
    __shared__ int32_t s_hist[kMaxExperts];
    __shared__ int32_t s_rank[kMaxRanks];
    __shared__ int16_t s_rank_of[kMaxExperts];
    __shared__ uint64_t s_bal[kGroups * kMaxRanks];
    __shared__ int32_t s_gpre[kGroups * kMaxRanks];
    __shared__ int32_t s_off[kMaxRanks + 1];
    __shared__ int32_t s_wsum[kGroups];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int nt = (int)T;  // 1 <= T <= kLayoutTile
    const bool writer = blockIdx.x == 0;
    const unsigned m0 = gridDim.x > 1 ? 1u : 0u;  // blocks m0.. move the rows
    const int lshift = (L & (L - 1)) == 0 ? __builtin_ctz(L) : -1;

    // this wave's items: token (-1: none) and the lane's vector of the chunk
    int it[kNormalFusedItems], iv[kNormalFusedItems];
    {
        const unsigned nbm = gridDim.x - m0;
        const unsigned w0 = (blockIdx.x - m0) * kGroups + __builtin_amdgcn_readfirstlane(tid / kWave);
#pragma unroll
        for (int j = 0; j < kNormalFusedItems; ++j) {
            const unsigned item = w0 + (unsigned)j * nbm * kGroups;
            const unsigned tj = item / (unsigned)ro.nchunk;
            it[j] = (blockIdx.x >= m0 && tj < (unsigned)nt) ? (int)tj : -1;
            iv[j] = (int)(item - tj * (unsigned)ro.nchunk) * kWave + lane;
        }
    }
    const bool direct = K <= kDirectTopk;
    int64_t raw[kMaxTopk];
    {
        const int64_t* tok = topk_idx + min(tid, nt - 1) * K;
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k) raw[k] = (direct && tid < nt && k < K) ? tok[k] : -1;
    }
    for (int i = tid; i < E; i += kLayoutTile) {
        s_hist[i] = 0;
        s_rank_of[i] = (int16_t)(i / L);
    }
    for (int i = tid; i < R; i += kLayoutTile) s_rank[i] = 0;
    if (!direct) stage_routing<kMaxTopk, kLayoutTile>(topk_idx, nt * K, E, s_idx);
    __syncthreads();
    uint4 buf[kNormalFusedItems];
    float wk[kNormalFusedItems];
    const bool with_topk = ro.recv_topk_idx != nullptr;
#pragma unroll
    for (int j = 0; j < kNormalFusedItems; ++j) {
        buf[j] = make_uint4(0, 0, 0, 0);
        if (it[j] >= 0 && iv[j] < ro.nvec) buf[j] = ro.x[(int64_t)it[j] * ro.nvec + iv[j]];
    }
#pragma unroll
    for (int j = 0; j < kNormalFusedItems; ++j) {
        wk[j] = 0.0f;
        if (with_topk && it[j] >= 0 && iv[j] < kWave && lane < K) wk[j] = ro.topk_w[(int64_t)it[j] * K + lane];
    }

    int e[kMaxTopk];
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
        if (direct)
            e[k] = (raw[k] >= 0 && raw[k] < E) ? (int)raw[k] : -1;
        else
            e[k] = (tid < nt && k < K) ? s_idx[tid * K + k] : -1;
    }
    if (direct && tid < nt)  // the rows' top-k metadata reads other tokens' slots
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k)
            if (k < K) s_idx[tid * K + k] = e[k];
    if (writer)
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k)
            if (e[k] >= 0) atomicAdd(&s_hist[e[k]], 1);
    uint64_t m[RW];
    token_rank_mask<RW>(e, s_rank_of, lshift, m);
    count_rank_tokens<RW>(m, R, s_rank, s_mask, s_bal);
    __syncthreads();
    // rows of each rank in earlier waves (group bases), then the rank offsets
    for (int r = tid; r < R; r += kLayoutTile) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < kGroups; ++w) {
            s_gpre[w * R + r] = run;
            run += __popcll(s_bal[w * R + r]);
        }
    }
    block_exclusive_scan2(R, [&](int r) { return s_rank[r]; }, s_off, s_wsum);
    __syncthreads();

    if (writer) {
        store_token_in_rank<RW, kLayoutTile>(m, s_mask, nt, R, itr);
        for (int i = tid; i < E; i += kLayoutTile) {
            ntpe[i] = s_hist[i];
            if (np.nrecv) np.nrecv[i] = (s_hist[i] + np.A - 1) / np.A * np.A;
        }
        for (int i = tid; i < R; i += kLayoutTile) {
            ntpr[i] = s_rank[i];
            np.tile_base[i] = 0;
        }
        for (int r = tid; r <= R; r += kLayoutTile) np.rank_offset[r] = s_off[r];
        const int gr = (nt + kWave - 1) / kWave * R;  // the plan's group words and bases, [groups, R]
        for (int i = tid; i < gr; i += kLayoutTile) {
            np.grp_bal[i] = s_bal[i];
            np.grp_pre[i] = s_gpre[i];
        }
    }
    {  // rows past the data carry no token, no expert and zero weights
        const int64_t n = min((int64_t)s_off[R], ro.cap);
        const int64_t stride = (int64_t)gridDim.x * kLayoutTile;
        const int64_t i0 = (int64_t)blockIdx.x * kLayoutTile + tid;
        for (int64_t r = n + i0; r < ro.cap; r += stride) ro.recv_src_idx[r] = -1;
        if (with_topk)
            for (int64_t i = n * K + i0; i < ro.cap * K; i += stride) {
                ro.recv_topk_idx[i] = -1;
                ro.recv_topk_w[i] = 0.0f;
            }
    }

#pragma unroll
    for (int j = 0; j < kNormalFusedItems; ++j) {
        const int t = it[j];
        if (t < 0) continue;
        const bool first = iv[j] < kWave;  // the token's chunk-0 item (wave-uniform)
        const int g = t / kWave;
        const int bitpos = t % kWave;
        const uint64_t below = (1ull << bitpos) - 1ull;
        int er = -1, el = -1;  // rank and rank-local id of this lane's slot
        if (first && with_topk && lane < K) {
            const int ex = s_idx[t * K + lane];
            if (ex >= 0) {
                er = lshift >= 0 ? ex >> lshift : ex / L;
                el = ex - er * L;
            }
        }
        const bool in = iv[j] < ro.nvec;  // whole 16-lane groups are in or out (H % 128 == 0 with CAST)
        uint2 code = make_uint2(0, 0);
        Fp8Scale sc{0.0f, 0.0f, 0u};
        if (CAST) {
            sc = fp8_block_scale(group16_max(in ? absmax_bf16x8(buf[j]) : 0.0f), ro.fmt);
            code = quantize_bf16x8(buf[j], sc.mul);
            if (in) {
                ro.xq[(int64_t)t * ro.nvec + iv[j]] = code;
                if ((lane & 15) == 0) {
                    const int64_t si = (int64_t)t * ro.nsb + iv[j] / 16;
                    if (ro.fmt == 2)
                        static_cast<uint8_t*>(ro.xs)[si] = (uint8_t)sc.ue8m0;
                    else
                        static_cast<float*>(ro.xs)[si] = sc.scale;
                }
            }
        }
        for (int rb = 0; rb < R; rb += kWave) {
            const int r = rb + lane;
            int d = -1;
            if (r < R) {
                const uint64_t b = s_bal[g * R + r];
                if ((b >> bitpos) & 1ull) {
                    const int64_t p = (int64_t)s_off[r] + s_gpre[g * R + r] + __popcll(b & below);
                    d = p < ro.cap ? (int)p : -1;
                }
                if (first) ro.send_row[(int64_t)t * R + r] = d;
            }
            uint64_t msk = ballot(d >= 0);
            while (msk) {
                const int jj = __builtin_ctzll(msk);
                msk &= msk - 1;
                const int dd = __shfl(d, jj, kWave);
                if (CAST) {
                    if (in) {
                        store_nt(ro.rq + (int64_t)dd * ro.nvec + iv[j], code);
                        if ((lane & 15) == 0) {
                            const int64_t si = (int64_t)dd * ro.nsb + iv[j] / 16;
                            if (ro.fmt == 2)
                                static_cast<uint8_t*>(ro.rs)[si] = (uint8_t)sc.ue8m0;
                            else
                                static_cast<float*>(ro.rs)[si] = sc.scale;
                        }
                    }
                } else if (in) {
                    store_nt(ro.recv_x + (int64_t)dd * ro.nvec + iv[j], buf[j]);
                }
                if (first) {
                    if (lane == 0) ro.recv_src_idx[dd] = t;
                    if (with_topk && lane < K) {
                        const bool on = er == rb + jj;
                        ro.recv_topk_idx[(int64_t)dd * K + lane] = on ? el : -1;
                        ro.recv_topk_w[(int64_t)dd * K + lane] = on ? wk[j] : 0.0f;
                    }
                }
            }
        }
    }
}

// get_dispatch_layout alone: the same tile work in blocks of TILE tokens,
// without a last-block handshake. Every block adds, for each expert and rank,
// (1 << 32) + its count to a 64-bit accumulator in the workspace with one
// device-scope atomic that returns the previous value: the high word counts
// the blocks that have added, the low word sums their counts (a total below
// 2^32, so no carry reaches the high word). The block whose add is the last
// one of a word (it finds gridDim.x - 1 blocks before it) holds that word's
// total: it writes the output and zeroes the word for the next call. So the
// counts are final one atomic round trip after the tile work, with no
// release / ticket / acquire sequence and no second pass over partials. The
// is_token_in_rank rows need no ordering with other blocks.
template <int RW, int TILE>
__global__ __launch_bounds__(TILE) void layout_acc_kernel(const int64_t* __restrict__ topk_idx, int64_t T, int K,
                                                          int E, int R, int L, int32_t* __restrict__ ntpr,
                                                          int32_t* __restrict__ ntpe, uint8_t* __restrict__ itr,
                                                          unsigned long long* __restrict__ acc) {
    __shared__ int32_t s_idx[TILE * kMaxTopk];
    __shared__ uint64_t s_mask[TILE * RW];
    __shared__ int32_t s_hist[kMaxExperts];
    __shared__ int32_t s_rank[kMaxRanks];
    __shared__ int16_t s_rank_of[kMaxExperts];

    const int tid = threadIdx.x;
    const int lshift = (L & (L - 1)) == 0 ? __builtin_ctz(L) : -1;
    const int64_t t0 = (int64_t)blockIdx.x * TILE;
    const int nt = (int)max<int64_t>(0, min<int64_t>(TILE, T - t0));

    // top-k <= kDirectTopk: each thread loads its own token's K entries (the
    // K loads of a wave together use every byte of the lines they touch),
    // in flight across the barrier that orders the LDS set-up before the
    // histogram, and no LDS round trip of the routing; larger top-k: the
    // coalesced stage through LDS
    const bool direct = K <= kDirectTopk;
    int64_t raw[kMaxTopk];
    const int64_t* tok = topk_idx + (t0 + min(tid, max(nt - 1, 0))) * K;
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) raw[k] = (direct && tid < nt && k < K) ? tok[k] : -1;
    for (int i = tid; i < E; i += TILE) {
        s_hist[i] = 0;
        s_rank_of[i] = (int16_t)(i / L);
    }
    for (int i = tid; i < R; i += TILE) s_rank[i] = 0;
    if (!direct) stage_routing<kMaxTopk, TILE>(topk_idx + t0 * K, nt * K, E, s_idx);
    __syncthreads();

    int e[kMaxTopk];
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
        if (direct)
            e[k] = (raw[k] >= 0 && raw[k] < E) ? (int)raw[k] : -1;
        else
            e[k] = (tid < nt && k < K) ? s_idx[tid * K + k] : -1;
    }
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k)
        if (e[k] >= 0) atomicAdd(&s_hist[e[k]], 1);
    uint64_t m[RW];
    token_rank_mask<RW>(e, s_rank_of, lshift, m);
    count_rank_tokens<RW>(m, R, s_rank, s_mask);
    __syncthreads();
    uint8_t* rows = itr + t0 * R;  // t0*R is a multiple of 16 when TILE is

    if (gridDim.x == 1) {
        for (int i = tid; i < E; i += TILE) ntpe[i] = s_hist[i];
        for (int i = tid; i < R; i += TILE) ntpr[i] = s_rank[i];
        store_token_in_rank<RW, TILE>(m, s_mask, nt, R, rows);
        return;
    }
    constexpr int kPer = (kMaxExperts + kMaxRanks + TILE - 1) / TILE;  // accumulator words per thread
    const unsigned long long one = 1ull << 32;
    unsigned long long prev[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {  // all adds in flight together
        const int i = tid + j * TILE;
        prev[j] = 0;
        if (i < E + R) {
            const int c = i < E ? s_hist[i] : s_rank[i - E];
            prev[j] = __hip_atomic_fetch_add(acc + i, one + (unsigned)c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    store_token_in_rank<RW, TILE>(m, s_mask, nt, R, rows);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = tid + j * TILE;
        if (i >= E + R || (unsigned)(prev[j] >> 32) != gridDim.x - 1) continue;
        const int total = (int)(unsigned)prev[j] + (i < E ? s_hist[i] : s_rank[i - E]);
        if (i < E)
            ntpe[i] = total;
        else
            ntpr[i - E] = total;
        __hip_atomic_store(acc + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

#ifndef CGD_LAYOUT_TILE
#define CGD_LAYOUT_TILE 512
#endif
constexpr int kLayoutAccTile = CGD_LAYOUT_TILE;  // tokens per block of get_dispatch_layout alone
static_assert(kLayoutAccTile % 16 == 0 && kLayoutAccTile % kWave == 0, "rows of a tile start 16-byte aligned");

int64_t layout_blocks(int64_t T) { return T <= 0 ? 1 : (T + kLayoutTile - 1) / kLayoutTile; }

size_t layout_partial_bytes(int64_t T, int E, int R) {
    const size_t arr = (size_t)layout_blocks(T) * (size_t)(E + R) * sizeof(int32_t);
    return kTicketBytes + (arr + 255) / 256 * 256;
}

size_t layout_workspace_bytes(int64_t, int E, int R) {
    return ((size_t)(E + R) * sizeof(unsigned long long) + 255) / 256 * 256;
}

hipError_t launch_layout(const int64_t* topk_idx, int64_t T, int K, int E, int R, int32_t* ntpr, int32_t* ntpe,
                         uint8_t* itr, void* workspace, hipStream_t stream) {
    unsigned long long* acc = reinterpret_cast<unsigned long long*>(workspace);
    constexpr int TILE = kLayoutAccTile;
    const dim3 grid((unsigned)(T <= 0 ? 1 : (T + TILE - 1) / TILE)), block(TILE);
    const int L = E / R;
    if (R <= 64)
        hipLaunchKernelGGL((layout_acc_kernel<1, TILE>), grid, block, 0, stream, topk_idx, T, K, E, R, L, ntpr, ntpe,
                           itr, acc);
    else
        hipLaunchKernelGGL((layout_acc_kernel<6, TILE>), grid, block, 0, stream, topk_idx, T, K, E, R, L, ntpr, ntpe,
                           itr, acc);
    return hipGetLastError();
}

hipError_t launch_layout_and_normal_plan(const int64_t* topk_idx, int64_t T, int K, int E, int R, int A,
                                         int32_t* ntpr, int32_t* ntpe, uint8_t* itr, int32_t* rank_offset,
                                         int32_t* nrecv, void* workspace, hipStream_t stream, const void* x,
                                         int64_t x_bytes, const NormalCast* cast) {
    // workspace: the rank-granular plan's workspace (its ticket, at offset 0
    // whatever the sizes, is the one this launch takes), then the block
    // partials
    NormalPlanArrays a = normal_plan_arrays(workspace, T, R);
    unsigned int* ticket = a.ticket;
    int32_t* partial = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + normal_workspace_bytes(T, R));
    const int nblk = (int)layout_blocks(T);
    const NormalPlanOut np{a.grp_bal, a.grp_pre, a.tile_base, rank_offset, nrecv, A};
    const int L = E / R;
    if (cast) {  // the spare blocks cast x (nothing to do for them in a one-tile plan: the caller casts)
        const CastOut co{cast->H, cast->fmt, reinterpret_cast<uint4*>(cast->q), cast->scales};
        const int extra = nblk > 1 ? kCastBlocks : 0;
        const dim3 grid((unsigned)(nblk + extra)), block(kLayoutTile);
        const uint4* xv = reinterpret_cast<const uint4*>(cast->x);
        if (R <= 64)
            hipLaunchKernelGGL((layout_kernel<1, true, true>), grid, block, 0, stream, topk_idx, T, K, E, R, L, ntpr,
                               ntpe, itr, partial, ticket, np, nblk, xv, 0, co);
        else
            hipLaunchKernelGGL((layout_kernel<6, true, true>), grid, block, 0, stream, topk_idx, T, K, E, R, L, ntpr,
                               ntpe, itr, partial, ticket, np, nblk, xv, 0, co);
        return hipGetLastError();
    }
    const uint4* pv = reinterpret_cast<const uint4*>(x);
    const int64_t pvecs = x ? x_bytes / 16 : 0;
    const int extra = (x && normal_plan_prefetches(T, x_bytes)) ? kPrefetchBlocks : 0;
    const dim3 grid((unsigned)(nblk + extra)), block(kLayoutTile);
    const CastOut none{0, 0, nullptr, nullptr};
    if (R <= 64)
        hipLaunchKernelGGL((layout_kernel<1, true>), grid, block, 0, stream, topk_idx, T, K, E, R, L, ntpr, ntpe, itr,
                           partial, ticket, np, nblk, pv, pvecs, none);
    else
        hipLaunchKernelGGL((layout_kernel<6, true>), grid, block, 0, stream, topk_idx, T, K, E, R, L, ntpr, ntpe, itr,
                           partial, ticket, np, nblk, pv, pvecs, none);
    return hipGetLastError();
}

hipError_t launch_layout_and_normal_fused(const void* x, int64_t T, int H, const int64_t* topk_idx,
                                          const float* topk_w, int K, int E, int R, int A, void* recv_x, int64_t cap,
                                          int32_t* ntpr, int32_t* ntpe, uint8_t* itr, int32_t* rank_offset,
                                          int32_t* nrecv, int32_t* recv_src_idx, int32_t* send_row,
                                          int64_t* recv_topk_idx, float* recv_topk_w, void* workspace,
                                          hipStream_t stream, const NormalCast* cast, void* recv_scales) {
    const NormalPlanArrays a = normal_plan_arrays(workspace, T, R);
    const NormalPlanOut np{a.grp_bal, a.grp_pre, a.tile_base, rank_offset, nrecv, A};
    const int nvec = H / 8;
    const int nchunk = (nvec + kWave - 1) / kWave;
    // one block per CU where that leaves at most kNormalFusedItems items per
    // wave (every block plans the tile in LDS: blocks sharing a CU would share
    // its LDS bandwidth for that); block 0 of a grid of several moves no rows
    constexpr int kWaves = kLayoutTile / kWave;
    const int64_t items = T * nchunk;
    const int64_t per_block = (int64_t)kWaves * kNormalFusedItems;
    const int64_t need = (items + per_block - 1) / per_block;
    const int64_t fill = (items + kWaves - 1) / kWaves;
    int64_t blocks = fill < device_cus() ? fill : device_cus();
    if (blocks < need) blocks = need;
    if (blocks > 1 && blocks < 1 + need) blocks = 1 + need;
    NormalRowsOut ro{reinterpret_cast<const uint4*>(x), nvec, nchunk, topk_w, reinterpret_cast<uint4*>(recv_x),
                     cap, send_row, recv_src_idx, recv_topk_idx, recv_topk_w, 0, 0, nullptr, nullptr, nullptr,
                     nullptr};
    if (cast) {  // recv_x holds the codes
        ro.recv_x = nullptr;
        ro.fmt = cast->fmt;
        ro.nsb = H / kFp8Block;
        ro.xq = reinterpret_cast<uint2*>(cast->q);
        ro.xs = cast->scales;
        ro.rq = reinterpret_cast<uint2*>(recv_x);
        ro.rs = recv_scales;
    }
    const dim3 grid((unsigned)(blocks < 1 ? 1 : blocks)), block(kLayoutTile);
#define CGD_NFUSED(RW, CAST)                                                                                         \
    hipLaunchKernelGGL((normal_fused_kernel<RW, CAST>), grid, block, 0, stream, topk_idx, T, K, E, R, E / R, ntpr, \
                       ntpe, itr, np, ro)
    if (R <= 64) {
        if (cast)
            CGD_NFUSED(1, true);
        else
            CGD_NFUSED(1, false);
    } else {
        if (cast)
            CGD_NFUSED(6, true);
        else
            CGD_NFUSED(6, false);
    }
#undef CGD_NFUSED
    return hipGetLastError();
}

hipError_t preload_layout() {
    hipFuncAttributes a;
    return hipFuncGetAttributes(&a, reinterpret_cast<const void*>(&layout_acc_kernel<1, kLayoutAccTile>));
}

}  // namespace cgd
