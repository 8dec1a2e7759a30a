// Rank-granular ("normal mode") dispatch and combine on gfx950.
//
// A token is received once by every rank that is_token_in_rank flags for it
// (DeepEP legacy test analysis page: normal-mode dispatch call, check_data
// walking the receive prefix sums, normal-mode combine check; DeepEP Python
// interface notes, "Dispatch API": recv_topk_idx, recv_topk_weights, aligned
// per-expert counts). Rank r's rows form one segment; segments follow in rank
// order and rows inside a segment follow ascending token order, the order in
// which one sender's tokens reach a rank.
//
//   normal_plan_kernel     one block per tile of 256 tokens. For every rank,
//                          each wave takes the ballot of its 64 tokens' flags
//                          (a "group word"); the block stores the group words,
//                          the rows of earlier groups of the tile, and the
//                          tile's per-rank count. The last block to finish
//                          turns tile counts into per-tile bases and the rank
//                          offsets (block scan).
//   normal_scatter_kernel  one wave per (token, column chunk). Lane r finds the
//                          token's row on rank r: rank offset + tile base +
//                          group base + popcount of the group word below the
//                          token. The chunk is loaded once and stored to every
//                          row with non-temporal stores; the token's chunk-0
//                          wave records send_row, recv_src_idx and each row's
//                          rank-local top-k ids and weights.
//   normal_combine_kernel  one wave per (token, column chunk): the token's rows
//                          in ascending rank order, gathered 8 at a time, are
//                          summed in fp32, then bias_0 and bias_1 are added,
//                          and the sum is rounded once to bf16. The chunk-0
//                          wave also sums the rows' top-k weights.
#include "cgd_device.h"
#include "cgd_launch.h"

namespace cgd {

#ifndef CGD_NORMAL_COMBINE_LDS
#define CGD_NORMAL_COMBINE_LDS (32 * 1024)
#endif
#ifndef CGD_NORMAL_COMBINE_LDS_WIDE
#define CGD_NORMAL_COMBINE_LDS_WIDE 54000
#endif
#ifndef CGD_NORMAL_COMBINE_U
#define CGD_NORMAL_COMBINE_U 2
#endif
#ifndef CGD_NORMAL_COMBINE_WAVES
#define CGD_NORMAL_COMBINE_WAVES 4
#endif
#ifndef CGD_NORMAL_GATHER
#define CGD_NORMAL_GATHER 8
#endif
#ifndef CGD_NORMAL_SCATTER_U
#define CGD_NORMAL_SCATTER_U 1
#endif
constexpr int kNormGroups = kRankTile / kWave;              // token groups (waves) per tile
constexpr int kFlagBatch = 16;                               // flag bytes in flight per thread
constexpr int kTileBatch = 16;                               // tile counts in flight per thread
constexpr int kNormScatterWaves = 4;                         // waves per scatter block
constexpr int kNormCombineWaves = CGD_NORMAL_COMBINE_WAVES;  // waves per combine block
constexpr int kGatherBatch = CGD_NORMAL_GATHER;              // rows in flight per combine wave
// Occupancy cap of the combine: an LDS reservation per block, 5 blocks per CU
// while a token has at most one gather batch of rows (min(K, R) <= 8), 3
// blocks above, where each wave keeps more rows in flight (top-16 over 64
// ranks: 703.5-703.9 us against 732.3-732.7 with 5 blocks; with 8 rows,
// prefill: 61.1 against 66.5).
constexpr size_t kNormCombineLds = CGD_NORMAL_COMBINE_LDS;
constexpr size_t kNormCombineLdsWide = CGD_NORMAL_COMBINE_LDS_WIDE;

// Normal workspace: ticket | group words u64 [G, R] | group bases int32 [G, R]
// | tile counts, then tile bases, int32 [tiles, R]; G = ceil(T / 64).
struct NormalWs {
    unsigned int* ticket;
    unsigned long long* grp_bal;
    int32_t* grp_pre;
    int32_t* tile_base;
};

static size_t round256(size_t b) { return (b + 255) / 256 * 256; }

static void normal_sizes(int64_t T, int R, int64_t* groups, int64_t* tiles) {
    const int64_t t = T > 0 ? T : 0;
    *groups = (t + kWave - 1) / kWave;
    *tiles = t > 0 ? (t + kRankTile - 1) / kRankTile : 1;
    (void)R;
}

size_t normal_workspace_bytes(int64_t T, int R) {
    int64_t G, tiles;
    normal_sizes(T, R, &G, &tiles);
    return kTicketBytes + round256((size_t)G * R * 8) + round256((size_t)G * R * 4) +
           round256((size_t)tiles * R * 4);
}

static NormalWs normal_ws(void* workspace, int64_t T, int R);

NormalPlanArrays normal_plan_arrays(void* workspace, int64_t T, int R) {
    const NormalWs w = normal_ws(workspace, T, R);
    return NormalPlanArrays{w.ticket, w.grp_bal, w.grp_pre, w.tile_base};
}

static NormalWs normal_ws(void* workspace, int64_t T, int R) {
    int64_t G, tiles;
    normal_sizes(T, R, &G, &tiles);
    char* p = reinterpret_cast<char*>(workspace);
    NormalWs w;
    w.ticket = reinterpret_cast<unsigned int*>(p);
    p += kTicketBytes;
    w.grp_bal = reinterpret_cast<unsigned long long*>(p);
    p += round256((size_t)G * R * 8);
    w.grp_pre = reinterpret_cast<int32_t*>(p);
    p += round256((size_t)G * R * 4);
    w.tile_base = reinterpret_cast<int32_t*>(p);
    return w;
}

__global__ __launch_bounds__(kRankTile) void normal_plan_kernel(const uint8_t* __restrict__ itr, int64_t T, int R,
                                                                const int32_t* __restrict__ ntpe,
                                                                int32_t* __restrict__ nrecv, int E, int A,
                                                                unsigned long long* __restrict__ grp_bal,
                                                                int32_t* __restrict__ grp_pre,
                                                                int32_t* __restrict__ tile_base,
                                                                int32_t* __restrict__ rank_offset,
                                                                unsigned int* __restrict__ ticket) {
    __shared__ unsigned long long s_bal[kNormGroups][kMaxRanks];
    __shared__ int32_t s_tot[kMaxRanks];
    __shared__ int32_t s_off[kMaxRanks + 1];
    __shared__ int32_t s_wsum[kNormGroups];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = lane_id();
    const int tile = blockIdx.x;
    const int ntiles = gridDim.x;
    const int64_t t = (int64_t)tile * kRankTile + tid;
    const bool mine = t < T;
    const int64_t G = (T + kWave - 1) / kWave;

    // per-expert receive counts rounded up to the alignment (elementwise)
    if (ntpe)
        for (int e = tile * kRankTile + tid; e < E; e += ntiles * kRankTile) nrecv[e] = (ntpe[e] + A - 1) / A * A;

    // ---- 1. group words: ballot of the 64 tokens' flags, rank by rank ----
    const uint8_t* row = itr + (mine ? t * R : 0);
    for (int r0 = 0; r0 < R; r0 += kFlagBatch) {
        uint8_t f[kFlagBatch];
#pragma unroll
        for (int j = 0; j < kFlagBatch; ++j) f[j] = (mine && r0 + j < R) ? row[r0 + j] : 0;
#pragma unroll
        for (int j = 0; j < kFlagBatch; ++j) {
            const uint64_t b = ballot(f[j] != 0);
            if (lane == 0 && r0 + j < R) s_bal[wave][r0 + j] = b;
        }
    }
    __syncthreads();
    // group bases inside the tile and the tile's per-rank count
    for (int r = tid; r < R; r += kRankTile) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < kNormGroups; ++w) {
            const int64_t g = (int64_t)tile * kNormGroups + w;
            const uint64_t b = s_bal[w][r];
            if (g < G) {
                grp_bal[g * R + r] = b;
                grp_pre[g * R + r] = run;
            }
            run += __popcll(b);
        }
        tile_base[(int64_t)tile * R + r] = run;
    }

    if (!last_block_done(ticket)) return;

    // ---- 2. last block: per-tile bases (one pass) and rank offsets ----
    for (int r = tid; r < R; r += kRankTile) {
        int run = 0;
        for (int b0 = 0; b0 < ntiles; b0 += kTileBatch) {
            int v[kTileBatch];
#pragma unroll
            for (int j = 0; j < kTileBatch; ++j) v[j] = (b0 + j < ntiles) ? tile_base[(int64_t)(b0 + j) * R + r] : 0;
#pragma unroll
            for (int j = 0; j < kTileBatch; ++j) {
                if (b0 + j < ntiles) tile_base[(int64_t)(b0 + j) * R + r] = run;
                run += v[j];
            }
        }
        s_tot[r] = run;
    }
    __syncthreads();
    block_exclusive_scan2(R, [&](int r) { return s_tot[r]; }, s_off, s_wsum);
    __syncthreads();
    for (int r = tid; r <= R; r += kRankTile) rank_offset[r] = s_off[r];
    reset_ticket(ticket);
}

// With CACHED the rows come from a stored send_row (cached dispatch) and no
// metadata is written. recv_topk_idx == nullptr: dispatch without top-k.
template <int U, bool CACHED>
__global__ __launch_bounds__(kNormScatterWaves* kWave) void normal_scatter_kernel(
    const uint4* __restrict__ x, int64_t T, int nvec, int nchunk, int R, const unsigned long long* __restrict__ grp_bal,
    const int32_t* __restrict__ grp_pre, const int32_t* __restrict__ tile_base, const int32_t* __restrict__ rank_offset,
    int32_t* __restrict__ send_row, int32_t* __restrict__ recv_src_idx, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int K, int E, int L, int64_t* __restrict__ recv_topk_idx,
    float* __restrict__ recv_topk_w, int64_t cap, int64_t t0, int fill, uint4* __restrict__ recv_x,
    SideRows side) {
    const int lane = lane_id();
    if (!CACHED && fill) {
        // rows past the data carry no token, no expert and zero weights
        const int64_t n = max<int64_t>(0, min<int64_t>(rank_offset[R], cap));
        const int64_t stride = (int64_t)gridDim.x * (kNormScatterWaves * kWave);
        const int64_t i0 = (int64_t)blockIdx.x * (kNormScatterWaves * kWave) + threadIdx.x;
        for (int64_t r = n + i0; r < cap; r += stride) recv_src_idx[r] = -1;
        if (recv_topk_idx)
            for (int64_t i = n * K + i0; i < cap * K; i += stride) {
                recv_topk_idx[i] = -1;
                recv_topk_w[i] = 0.0f;
            }
    }
    const int64_t g = (int64_t)blockIdx.x * kNormScatterWaves + threadIdx.x / kWave;
    const int64_t tr = g / nchunk;
    const int64_t t = t0 + tr;  // T is the end of this launch's token range
    if (t >= T) return;
    const int c = (int)(g - tr * nchunk);
    const int v0 = c * U * kWave;
    const uint4* xr = x + t * nvec;
    uint4 buf[U];  // loaded before the rows are known
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int v = v0 + u * kWave + lane;
        if (v < nvec) buf[u] = xr[v];
    }
    const bool meta = !CACHED && c == 0;
    const bool with_topk = meta && recv_topk_idx != nullptr;  // then topk_idx is given too (T > 0)
    int er = -1, el = -1;  // rank and rank-local id of this lane's slot
    float wk = 0.0f;
    if (with_topk && lane < K) {
        const int64_t e = topk_idx[t * K + lane];
        if (e >= 0 && e < E) {
            er = (int)e / L;
            el = (int)e - er * L;
        }
        wk = topk_w[t * K + lane];
    }
    const int64_t grp = t / kWave;
    const int64_t tile = t / kRankTile;
    const int bitpos = (int)(t % kWave);
    const uint64_t below = (1ull << bitpos) - 1ull;
    for (int rb = 0; rb < R; rb += kWave) {
        const int r = rb + lane;
        int d = -1;
        if (r < R) {
            if (CACHED) {
                const int p = send_row[t * R + r];
                d = (p >= 0 && p < cap) ? p : -1;
            } else {
                const uint64_t b = grp_bal[grp * R + r];
                if ((b >> bitpos) & 1ull) {
                    const int64_t p = (int64_t)rank_offset[r] + tile_base[tile * R + r] + grp_pre[grp * R + r] +
                                      __popcll(b & below);
                    // only a malformed is_token_in_rank (or workspace) leaves [0, cap)
                    d = (p >= 0 && p < cap) ? (int)p : -1;
                }
                if (c == 0) send_row[t * R + r] = d;
            }
        }
        uint64_t m = ballot(d >= 0);
        while (m) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            const int dd = __shfl(d, j, kWave);
            uint4* dr = recv_x + (int64_t)dd * nvec;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * kWave + lane;
                if (v < nvec) store_nt(dr + v, buf[u]);
            }
            if (side.src && c == 0) copy_side_row(side, t, dd, lane);
            if (meta) {
                if (lane == 0) recv_src_idx[dd] = (int32_t)t;
                if (with_topk && lane < K) {
                    const bool on = er == rb + j;
                    recv_topk_idx[(int64_t)dd * K + lane] = on ? el : -1;
                    recv_topk_w[(int64_t)dd * K + lane] = on ? wk : 0.0f;
                }
            }
        }
    }
}

template <int U>
__global__ __launch_bounds__(kNormCombineWaves* kWave) void normal_combine_kernel(
    const uint4* __restrict__ y, int64_t rows, int nvec, int nchunk, const int32_t* __restrict__ send_row, int R,
    int64_t T, const float* __restrict__ recv_w, int K, const uint4* __restrict__ bias0,
    const uint4* __restrict__ bias1, uint4* __restrict__ out, float* __restrict__ out_w) {
    const int lane = lane_id();
    const int64_t g = (int64_t)blockIdx.x * kNormCombineWaves + threadIdx.x / kWave;
    const int64_t t = g / nchunk;
    if (t >= T) return;
    const int c = (int)(g - t * nchunk);
    const int v0 = c * U * kWave;
    const bool wsum_here = out_w != nullptr && c == 0 && lane < K;

    uint4 b0[U], b1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int v = v0 + u * kWave + lane;
        if (bias0 && v < nvec) b0[u] = load_nt(bias0 + t * nvec + v);
        if (bias1 && v < nvec) b1[u] = load_nt(bias1 + t * nvec + v);
    }
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
    float wsum = 0.0f;

    for (int rb = 0; rb < R; rb += kWave) {
        const int r = rb + lane;
        int d = -1;
        if (r < R) {
            const int p = send_row[t * R + r];
            d = (p >= 0 && p < rows) ? p : -1;
        }
        uint64_t m = ballot(d >= 0);
        while (m) {
            int dk[kGatherBatch];
#pragma unroll
            for (int i = 0; i < kGatherBatch; ++i) {
                dk[i] = -1;
                if (m) {
                    dk[i] = __shfl(d, __builtin_ctzll(m), kWave);
                    m &= m - 1;
                }
            }
            uint4 q[kGatherBatch][U];
#pragma unroll
            for (int i = 0; i < kGatherBatch; ++i) {
                if (dk[i] < 0) continue;
                const uint4* yr = y + (int64_t)dk[i] * nvec;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int v = v0 + u * kWave + lane;
                    if (v < nvec) q[i][u] = load_nt(yr + v);
                }
            }
            float wv[kGatherBatch];
            if (wsum_here)
#pragma unroll
                for (int i = 0; i < kGatherBatch; ++i) wv[i] = dk[i] >= 0 ? recv_w[(int64_t)dk[i] * K + lane] : 0.0f;
#pragma unroll
            for (int i = 0; i < kGatherBatch; ++i) {
                if (dk[i] < 0) continue;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint4 s = q[i][u];
                    acc[u][0] += bf16_lo(s.x);
                    acc[u][1] += bf16_hi(s.x);
                    acc[u][2] += bf16_lo(s.y);
                    acc[u][3] += bf16_hi(s.y);
                    acc[u][4] += bf16_lo(s.z);
                    acc[u][5] += bf16_hi(s.z);
                    acc[u][6] += bf16_lo(s.w);
                    acc[u][7] += bf16_hi(s.w);
                }
                if (wsum_here) wsum += wv[i];
            }
        }
    }

    uint4* orow = out + t * nvec;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int v = v0 + u * kWave + lane;
        if (v >= nvec) continue;
        float* a = acc[u];
        if (bias0) {
            const uint4 s = b0[u];
            a[0] += bf16_lo(s.x), a[1] += bf16_hi(s.x), a[2] += bf16_lo(s.y), a[3] += bf16_hi(s.y);
            a[4] += bf16_lo(s.z), a[5] += bf16_hi(s.z), a[6] += bf16_lo(s.w), a[7] += bf16_hi(s.w);
        }
        if (bias1) {
            const uint4 s = b1[u];
            a[0] += bf16_lo(s.x), a[1] += bf16_hi(s.x), a[2] += bf16_lo(s.y), a[3] += bf16_hi(s.y);
            a[4] += bf16_lo(s.z), a[5] += bf16_hi(s.z), a[6] += bf16_lo(s.w), a[7] += bf16_hi(s.w);
        }
        uint4 o;
        o.x = pack_bf16x2(a[0], a[1]);
        o.y = pack_bf16x2(a[2], a[3]);
        o.z = pack_bf16x2(a[4], a[5]);
        o.w = pack_bf16x2(a[6], a[7]);
        store_nt(orow + v, o);
    }
    if (wsum_here) out_w[t * K + lane] = wsum;
}

// Chunks of 4 vectors per lane unless that leaves fewer than this many waves.
constexpr int64_t kNormMinWaves = 4096;

// The apply after a plan that pulled x into the caches runs fewer waves per
// CU: an LDS reservation of this many bytes per 4-wave block leaves 5 blocks.
// Whole rank-granular dispatch (layout + plan + apply), inputs rotating, us:
// prefill 68.9 against 69.7-69.9 at full occupancy (6 blocks 66.0, 4 blocks
// 68.8, 3 blocks 94.7), Zipf-skewed 171.5 against 184.5-184.7 (6 blocks
// 178.8, 4 blocks 171.5, 3 blocks 234.4).
#ifndef CGD_NORMAL_PF_LDS
#define CGD_NORMAL_PF_LDS 32768
#endif
template <bool CACHED, int U>
static void launch_normal_scatter_u(const void* x, int64_t T, int nvec, int R, const NormalWs* w,
                                    const int32_t* rank_offset, int32_t* send_row, int32_t* recv_src_idx,
                                    const int64_t* topk_idx, const float* topk_w, int K, int E,
                                    int64_t* recv_topk_idx, float* recv_topk_w, int64_t cap, void* recv_x,
                                    const SideRows& side, hipStream_t s, size_t lds = 0) {
    const int nchunk = (nvec + U * kWave - 1) / (U * kWave);
    const int64_t tper = tokens_per_launch(nchunk);
    int64_t t0 = 0;
    do {  // token ranges within 32-bit work-item ids; only the first fills the tail
        const int64_t nt = T - t0 < tper ? T - t0 : tper;
        const int64_t waves = nt * nchunk;
        const int64_t blocks = waves <= 0 ? 1 : (waves + kNormScatterWaves - 1) / kNormScatterWaves;
        hipLaunchKernelGGL((normal_scatter_kernel<U, CACHED>), dim3((unsigned)blocks),
                           dim3(kNormScatterWaves * kWave), lds, s, reinterpret_cast<const uint4*>(x), t0 + nt, nvec,
                           nchunk, R, w ? w->grp_bal : nullptr, w ? w->grp_pre : nullptr,
                           w ? w->tile_base : nullptr, rank_offset, send_row, recv_src_idx, topk_idx, topk_w, K, E,
                           R > 0 ? E / R : 1, recv_topk_idx, recv_topk_w, cap, t0, t0 == 0 ? 1 : 0,
                           reinterpret_cast<uint4*>(recv_x), side);
        t0 += tper;
    } while (t0 < T);
}

template <bool CACHED>
static void launch_normal_scatter(const void* x, int64_t T, int nvec, int R, const NormalWs* w,
                                  const int32_t* rank_offset, int32_t* send_row, int32_t* recv_src_idx,
                                  const int64_t* topk_idx, const float* topk_w, int K, int E, int64_t* recv_topk_idx,
                                  float* recv_topk_w, int64_t cap, void* recv_x, const SideRows& side,
                                  hipStream_t s, size_t lds = 0) {
    constexpr int U = CGD_NORMAL_SCATTER_U;
    const int64_t wavesU = T * ((nvec + U * kWave - 1) / (U * kWave));
    if (wavesU >= kNormMinWaves)
        launch_normal_scatter_u<CACHED, U>(x, T, nvec, R, w, rank_offset, send_row, recv_src_idx, topk_idx, topk_w,
                                           K, E, recv_topk_idx, recv_topk_w, cap, recv_x, side, s, lds);
    else
        launch_normal_scatter_u<CACHED, 1>(x, T, nvec, R, w, rank_offset, send_row, recv_src_idx, topk_idx, topk_w,
                                           K, E, recv_topk_idx, recv_topk_w, cap, recv_x, side, s);
}

static SideRows normal_no_side() { return SideRows{nullptr, 0, 0, 0, 0, nullptr}; }

hipError_t launch_normal_plan(const uint8_t* itr, int64_t T, int R, const int32_t* ntpe, int E, int A,
                              int32_t* rank_offset, int32_t* nrecv, void* workspace, hipStream_t stream) {
    const NormalWs w = normal_ws(workspace, T, R);
    int64_t G, tiles;
    normal_sizes(T, R, &G, &tiles);
    hipLaunchKernelGGL(normal_plan_kernel, dim3((unsigned)tiles), dim3(kRankTile), 0, stream, itr, T, R, ntpe, nrecv,
                       E, A, w.grp_bal, w.grp_pre, w.tile_base, rank_offset, w.ticket);
    return hipGetLastError();
}

hipError_t launch_normal_apply(const void* x, int64_t T, int H, const int64_t* topk_idx, const float* topk_w, int K,
                               int E, int R, void* recv_x, int64_t cap, const int32_t* rank_offset,
                               int32_t* recv_src_idx, int32_t* send_row, int64_t* recv_topk_idx, float* recv_topk_w,
                               const void* workspace, hipStream_t stream, bool after_prefetch) {
    const NormalWs w = normal_ws(const_cast<void*>(workspace), T, R);
    launch_normal_scatter<false>(x, T, H / 8, R, &w, rank_offset, send_row, recv_src_idx, topk_idx, topk_w, K, E,
                                 recv_topk_idx, recv_topk_w, cap, recv_x, normal_no_side(), stream,
                                 after_prefetch ? CGD_NORMAL_PF_LDS : 0);
    return hipGetLastError();
}

hipError_t launch_normal_apply_fp8(const void* xq, const void* xs, int64_t st, int64_t sb, int fmt, int64_t T, int H,
                                   const int64_t* topk_idx, const float* topk_w, int K, int E, int R, void* recv_q,
                                   void* recv_s, int64_t cap, const int32_t* rank_offset, int32_t* recv_src_idx,
                                   int32_t* send_row, int64_t* recv_topk_idx, float* recv_topk_w,
                                   const void* workspace, hipStream_t stream) {
    const NormalWs w = normal_ws(const_cast<void*>(workspace), T, R);
    const SideRows side{xs, st, sb, H / kFp8Block, fmt == 2 ? 1 : 4, recv_s};
    launch_normal_scatter<false>(xq, T, H / 16, R, &w, rank_offset, send_row, recv_src_idx, topk_idx, topk_w, K, E,
                                 recv_topk_idx, recv_topk_w, cap, recv_q, side, stream);
    return hipGetLastError();
}

hipError_t launch_normal_dispatch_cached(const void* x, int64_t T, int H, int R, const int32_t* send_row,
                                         void* recv_x, int64_t cap, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    launch_normal_scatter<true>(x, T, H / 8, R, nullptr, nullptr, const_cast<int32_t*>(send_row), nullptr, nullptr,
                                nullptr, 1, 1, nullptr, nullptr, cap, recv_x, normal_no_side(), stream);
    return hipGetLastError();
}

hipError_t launch_normal_dispatch_cached_fp8(const void* xq, const void* xs, int64_t st, int64_t sb, int fmt,
                                             int64_t T, int H, int R, const int32_t* send_row, void* recv_q,
                                             void* recv_s, int64_t cap, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const SideRows side{xs, st, sb, H / kFp8Block, fmt == 2 ? 1 : 4, recv_s};
    launch_normal_scatter<true>(xq, T, H / 16, R, nullptr, nullptr, const_cast<int32_t*>(send_row), nullptr, nullptr,
                                nullptr, 1, 1, nullptr, nullptr, cap, recv_q, side, stream);
    return hipGetLastError();
}

hipError_t launch_normal_combine(const void* expert_out, int64_t rows, int H, const int32_t* send_row, int64_t T,
                                 int R, const float* recv_w, int K, const void* bias0, const void* bias1, void* out,
                                 float* out_w, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    constexpr int U = CGD_NORMAL_COMBINE_U;
    const int nvec = H / 8;
    const int nchunk = (nvec + U * kWave - 1) / (U * kWave);
    const int64_t tper = tokens_per_launch(nchunk);
    const size_t lds = (K < R ? K : R) > kGatherBatch ? kNormCombineLdsWide : kNormCombineLds;
    for (int64_t t0 = 0; t0 < T; t0 += tper) {  // token ranges; the kernel indexes tokens relative to its pointers
        const int64_t nt = T - t0 < tper ? T - t0 : tper;
        const int64_t blocks = (nt * nchunk + kNormCombineWaves - 1) / kNormCombineWaves;
        const uint4* b0 = bias0 ? reinterpret_cast<const uint4*>(bias0) + t0 * nvec : nullptr;
        const uint4* b1 = bias1 ? reinterpret_cast<const uint4*>(bias1) + t0 * nvec : nullptr;
        hipLaunchKernelGGL((normal_combine_kernel<U>), dim3((unsigned)blocks), dim3(kNormCombineWaves * kWave),
                           lds, stream, reinterpret_cast<const uint4*>(expert_out), rows, nvec, nchunk,
                           send_row + t0 * R, R, nt, recv_w, K, b0, b1, reinterpret_cast<uint4*>(out) + t0 * nvec,
                           out_w ? out_w + t0 * K : nullptr);
    }
    return hipGetLastError();
}

hipError_t preload_normal() {
    hipFuncAttributes a;
    return hipFuncGetAttributes(&a, reinterpret_cast<const void*>(&normal_plan_kernel));
}

}  // namespace cgd
