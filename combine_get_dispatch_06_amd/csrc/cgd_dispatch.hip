// Dispatch permutation on gfx950.
//
// Every selected (token, slot) pair gets one row of its expert's receive
// segment; segments are laid end to end in ascending expert id, each sized to
// its row count rounded up to expert_alignment (DeepEP Python interface notes,
// "Dispatch API": expert_alignment, the receive buffer and the handle). Inside
// a segment, rows follow ascending (token, slot), which makes the permutation
// unique and independent of scheduling.
//
// Two launches:
//   rank_kernel     one block per tile of 256 tokens (4 waves, one token per
//                   lane). For each slot it finds the number of earlier slots
//                   of the tile with the same expert: inside a wave with
//                   wavefront ballots (a "multi-split": lanes whose expert
//                   agrees with mine on every bit of the expert id are my
//                   peers; popcount of the peers below my lane), across the
//                   tile's waves with an LDS histogram and a prefix over
//                   waves. It writes the tile's expert histogram and a packed
//                   (expert, rank-in-tile) word per slot. The last block to
//                   finish turns the tile histograms into per-tile bases
//                   (column prefix over tiles), computes the aligned segment
//                   offsets with a block prefix scan, and marks padding rows.
//   scatter_kernel  one wave per token: lanes 0..K-1 turn their slot into a
//                   final row (tile base + rank-in-tile), record dst_row and
//                   recv_src_idx, then the whole wave streams the token's row
//                   through registers in 16-byte vectors and stores it to the
//                   K destination rows with non-temporal stores. The row is
//                   read from HBM once however many experts it goes to.
// Cached dispatch runs scatter_kernel alone on a stored dst_row.
#include "cgd_device.h"
#include "cgd_launch.h"

namespace cgd {

constexpr int kRankWaves = kRankTile / kWave;
constexpr int kPackBits = 13;  // rank inside a tile < 256 * 16 = 4096 < 2^13
constexpr int kScatterWaves = 4;

template <int KT>
__global__ __launch_bounds__(kRankTile) void rank_kernel(const int64_t* __restrict__ topk_idx, int64_t T, int E,
                                                         int ebits, int A, int32_t* __restrict__ dst_row,
                                                         int32_t* __restrict__ tile_base,
                                                         int32_t* __restrict__ expert_offset,
                                                         int32_t* __restrict__ recv_src_idx,
                                                         unsigned int* __restrict__ ticket) {
    __shared__ int32_t s_idx[kRankTile * KT];
    __shared__ int32_t s_wh[kRankWaves][kMaxExperts];
    __shared__ int32_t s_off[kMaxExperts + 1];
    __shared__ int32_t s_wsum[kRankWaves];

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = lane_id();
    const int64_t t0 = (int64_t)blockIdx.x * kRankTile;
    const int nt = (int)max<int64_t>(0, min<int64_t>(kRankTile, T - t0));

    for (int i = tid; i < kRankWaves * kMaxExperts; i += kRankTile) (&s_wh[0][0])[i] = 0;
    {
        const int64_t* src = topk_idx + t0 * KT;
        const int n = nt * KT;
        for (int i = tid; i < n; i += kRankTile) {
            const int64_t e = src[i];
            s_idx[i] = (e >= 0 && e < E) ? (int32_t)e : -1;
        }
    }
    __syncthreads();

    int e[KT], rk[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        e[k] = (tid < nt) ? s_idx[tid * KT + k] : -1;
        rk[k] = 0;
    }

    // rank inside the wave: earlier lanes (tokens) holding my expert in any
    // slot, plus earlier slots of my own token holding it
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int kp = 0; kp < KT; ++kp) {
        const uint64_t valid = ballot(e[kp] >= 0);
        uint64_t bits[10];
#pragma unroll
        for (int b = 0; b < 10; ++b) bits[b] = (b < ebits) ? ballot((e[kp] >> b) & 1) : 0ull;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            uint64_t peers = valid;
#pragma unroll
            for (int b = 0; b < 10; ++b)
                if (b < ebits) peers &= ((e[k] >> b) & 1) ? bits[b] : ~bits[b];
            rk[k] += __popcll(peers & lt) + ((kp < k && e[kp] == e[k]) ? 1 : 0);
        }
    }

#pragma unroll
    for (int k = 0; k < KT; ++k)
        if (e[k] >= 0) atomicAdd(&s_wh[wave][e[k]], 1);
    __syncthreads();

    // per expert: prefix over the tile's waves; the total is the tile histogram
    for (int x = tid; x < E; x += kRankTile) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < kRankWaves; ++w) {
            const int c = s_wh[w][x];
            s_wh[w][x] = run;
            run += c;
        }
        tile_base[(int64_t)blockIdx.x * E + x] = run;
    }
    __syncthreads();

    // packed (expert, rank-in-tile) per slot, staged in LDS for coalesced stores
#pragma unroll
    for (int k = 0; k < KT; ++k)
        if (tid < nt) s_idx[tid * KT + k] = (e[k] >= 0) ? ((e[k] << kPackBits) | (s_wh[wave][e[k]] + rk[k])) : -1;
    __syncthreads();
    {
        int32_t* out = dst_row + t0 * KT;
        const int n = nt * KT;
        for (int i = tid; i < n; i += kRankTile) out[i] = s_idx[i];
    }

    if (!last_block_done(ticket)) return;

    // ---- last block: tile bases, segment offsets, padding rows ----
    const int ntiles = gridDim.x;
    // 1. rows per expert = sum of the tile histograms
    for (int x = tid; x < E; x += kRankTile) {
        int s = 0;
        for (int b = 0; b < ntiles; ++b) s += tile_base[(int64_t)b * E + x];
        s_wh[0][x] = s;
    }
    __syncthreads();
    // 2. exclusive scan of the aligned sizes: thread i owns entries 2i, 2i+1
    {
        const int i0 = 2 * tid, i1 = 2 * tid + 1;
        const int c0 = (i0 < E) ? (s_wh[0][i0] + A - 1) / A * A : 0;
        const int c1 = (i1 < E) ? (s_wh[0][i1] + A - 1) / A * A : 0;
        const int own = c0 + c1;
        int inc = own;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int v = __shfl_up(inc, d, kWave);
            if (lane >= d) inc += v;
        }
        if (lane == kWave - 1) s_wsum[wave] = inc;
        __syncthreads();
        int before = 0;
        for (int w = 0; w < wave; ++w) before += s_wsum[w];
        const int excl = before + inc - own;
        if (i0 < E) s_off[i0] = excl;
        if (i1 < E) s_off[i1] = excl + c0;
        if (tid == kRankTile - 1) s_off[E] = before + inc;  // entries >= E add 0
    }
    __syncthreads();
    // 3. per-tile bases (segment offset + rows of earlier tiles), padding rows
    for (int x = tid; x < E; x += kRankTile) {
        int run = s_off[x];
        for (int b = 0; b < ntiles; ++b) {
            int32_t* p = tile_base + (int64_t)b * E + x;
            const int h = *p;
            *p = run;
            run += h;
        }
        for (int r = run; r < s_off[x + 1]; ++r) recv_src_idx[r] = -1;
    }
    for (int x = tid; x <= E; x += kRankTile) expert_offset[x] = s_off[x];
    reset_ticket(ticket);
}

// One wave per token. PACKED: dst_row holds rank_kernel's packed words and is
// rewritten with final rows (non-cached dispatch); otherwise dst_row holds
// final rows and is only read (cached dispatch).
template <int KM, int U, bool PACKED>
__global__ __launch_bounds__(kScatterWaves* kWave) void scatter_kernel(
    const uint4* __restrict__ x, int64_t T, int nvec, int K, int32_t* __restrict__ dst_row,
    const int32_t* __restrict__ tile_base, int E, int32_t* __restrict__ recv_src_idx,
    const int32_t* __restrict__ expert_offset, int64_t cap, uint4* __restrict__ recv_x) {
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();

    if (PACKED) {
        // rows past the data carry no source token
        const int64_t n = expert_offset[E];
        const int64_t stride = (int64_t)gridDim.x * blockDim.x;
        for (int64_t r = n + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < cap; r += stride)
            recv_src_idx[r] = -1;
    }

    const int64_t t = (int64_t)blockIdx.x * kScatterWaves + wave;
    if (t >= T) return;

    int d = -1;
    if (lane < K) {
        const int p = dst_row[t * K + lane];
        if (PACKED) {
            if (p >= 0) {
                const int ex = p >> kPackBits;
                const int lr = p & ((1 << kPackBits) - 1);
                d = tile_base[(t / kRankTile) * E + ex] + lr;
                if (d >= cap) d = -1;  // cannot happen for a consistent workspace; never write outside recv_x
                if (d >= 0) recv_src_idx[d] = (int32_t)t;
            }
            dst_row[t * K + lane] = d;
        } else {
            d = (p >= 0 && p < cap) ? p : -1;
        }
    }
    int dk[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) dk[k] = __shfl(d, k, kWave);

    const uint4* xr = x + t * nvec;
    for (int v0 = 0; v0 < nvec; v0 += U * kWave) {
        uint4 buf[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kWave + lane;
            if (v < nvec) buf[u] = xr[v];
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
        }
    }
}

size_t dispatch_workspace_bytes(int64_t T, int E) {
    const int64_t ntiles = T <= 0 ? 1 : (T + kRankTile - 1) / kRankTile;
    const size_t arr = (size_t)ntiles * (size_t)E * sizeof(int32_t);
    return kTicketBytes + (arr + 255) / 256 * 256;
}

template <int KT>
static void launch_rank(dim3 grid, hipStream_t s, const int64_t* idx, int64_t T, int E, int ebits, int A,
                        int32_t* dst_row, int32_t* tile_base, int32_t* off, int32_t* src, unsigned int* ticket) {
    hipLaunchKernelGGL(rank_kernel<KT>, grid, dim3(kRankTile), 0, s, idx, T, E, ebits, A, dst_row, tile_base, off,
                       src, ticket);
}

template <bool PACKED>
static void launch_scatter(int64_t T, int K, hipStream_t s, const void* x, int nvec, int32_t* dst_row,
                           const int32_t* tile_base, int E, int32_t* src, const int32_t* off, int64_t cap,
                           void* recv_x) {
    const int64_t blocks = T <= 0 ? 1 : (T + kScatterWaves - 1) / kScatterWaves;
    const dim3 grid((unsigned)blocks), block(kScatterWaves * kWave);
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    uint4* rv = reinterpret_cast<uint4*>(recv_x);
#define CGD_SCATTER(KM, U) \
    hipLaunchKernelGGL((scatter_kernel<KM, U, PACKED>), grid, block, 0, s, xv, T, nvec, K, dst_row, tile_base, E, \
                       src, off, cap, rv)
    if (K <= 2)
        CGD_SCATTER(2, 8);
    else if (K <= 4)
        CGD_SCATTER(4, 8);
    else if (K <= 8)
        CGD_SCATTER(8, 8);
    else
        CGD_SCATTER(16, 8);
#undef CGD_SCATTER
}

hipError_t launch_dispatch(const void* x, int64_t T, int H, const int64_t* topk_idx, int K, int E, int A,
                           void* recv_x, int64_t cap, int32_t* expert_offset, int32_t* recv_src_idx,
                           int32_t* dst_row, void* workspace, hipStream_t stream) {
    unsigned int* ticket = reinterpret_cast<unsigned int*>(workspace);
    int32_t* tile_base = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + kTicketBytes);
    const dim3 grid((unsigned)(T <= 0 ? 1 : (T + kRankTile - 1) / kRankTile));
    int ebits = 0;
    while ((1 << ebits) < E) ++ebits;
    switch (K) {
#define CGD_RANK_CASE(KT) \
    case KT:              \
        launch_rank<KT>(grid, stream, topk_idx, T, E, ebits, A, dst_row, tile_base, expert_offset, recv_src_idx, ticket); \
        break;
        CGD_RANK_CASE(1) CGD_RANK_CASE(2) CGD_RANK_CASE(3) CGD_RANK_CASE(4)
        CGD_RANK_CASE(5) CGD_RANK_CASE(6) CGD_RANK_CASE(7) CGD_RANK_CASE(8)
        CGD_RANK_CASE(9) CGD_RANK_CASE(10) CGD_RANK_CASE(11) CGD_RANK_CASE(12)
        CGD_RANK_CASE(13) CGD_RANK_CASE(14) CGD_RANK_CASE(15) CGD_RANK_CASE(16)
#undef CGD_RANK_CASE
        default:
            return hipErrorInvalidValue;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    launch_scatter<true>(T, K, stream, x, H / 8, dst_row, tile_base, E, recv_src_idx, expert_offset, cap, recv_x);
    return hipGetLastError();
}

hipError_t launch_dispatch_cached(const void* x, int64_t T, int H, int K, const int32_t* dst_row, void* recv_x,
                                  int64_t cap, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    launch_scatter<false>(T, K, stream, x, H / 8, const_cast<int32_t*>(dst_row), nullptr, 0, nullptr, nullptr, cap,
                          recv_x);
    return hipGetLastError();
}

}  // namespace cgd
