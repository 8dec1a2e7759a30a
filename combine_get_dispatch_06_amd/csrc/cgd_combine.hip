// Weighted combine on gfx950.
//
// combined_x[t] = bf16( sum over selected slots k, ascending, of
//                       w[t,k] * expert_out[dst_row[t,k]] )
// (DeepEP legacy test analysis page, low-latency combine check: the result is
// x scaled by the sum of the unmasked weights when experts are identities).
//
// Work is split into (token, column chunk) items, a chunk being 64*U
// 16-byte vectors (1 KB per U) of the row, one wave each; blocks start in
// item order, so the gathers in flight stay close together. Residency is
// capped by an LDS reservation per block: 5 blocks of 4 waves per CU up to
// top-8, 3 blocks above (each wave then has twice the loads in flight); fewer
// concurrent gathers per CU and many short items measured faster than one
// long-lived wave per token or full occupancy. Top-16, hidden 4096 (32768
// tokens): 758 us at 8-12 waves per CU against 778-781 at 14 and 794 at 20;
// top-8 at hidden 7168: 88 us at 20 waves against 97 at 12.
// Lanes 0..K-1 read the token's K rows and weights and broadcast them; each
// lane then issues its K*U gathered 16-byte loads before any arithmetic,
// accumulates in fp32 with fused multiply-add in ascending k from +0,
// converts to bf16 with round to nearest even, and writes its chunk once.
// Expert rows are read with non-temporal loads (each is read exactly once).
#include "cgd_device.h"
#include "cgd_launch.h"

namespace cgd {

#ifndef CGD_COMBINE_WAVES
#define CGD_COMBINE_WAVES 4
#endif
#ifndef CGD_COMBINE_U
#define CGD_COMBINE_U 1
#endif
// Occupancy cap: each block reserves this much (unused) LDS, so at most
// 160 KB / CGD_COMBINE_LDS_CAP blocks share a CU (5 at 32 KB);
// CGD_COMBINE_LDS_WIDE is the reservation for top-k above 8 (3 at 54000 B).
#ifndef CGD_COMBINE_LDS_CAP
#define CGD_COMBINE_LDS_CAP (32 * 1024)
#endif
#ifndef CGD_COMBINE_LDS_WIDE
#define CGD_COMBINE_LDS_WIDE 54000
#endif
constexpr int kCombineWaves = CGD_COMBINE_WAVES;  // waves per block

template <int KM, int U>
__global__ __launch_bounds__(kCombineWaves* kWave) void combine_kernel(const uint4* __restrict__ y, int64_t cap,
                                                                        int nvec, int nchunk,
                                                                        const int32_t* __restrict__ dst_row,
                                                                        const float* __restrict__ w, int64_t T, int K,
                                                                        uint4* __restrict__ out) {
    const int lane = lane_id();
    const int64_t g = (int64_t)blockIdx.x * kCombineWaves + threadIdx.x / kWave;
    {
        const int64_t t = g / nchunk;
        if (t >= T) return;
        const int v0 = (int)(g - t * nchunk) * (U * kWave);

        int d = -1;
        float wt = 0.0f;
        if (lane < K) {
            const int p = dst_row[t * K + lane];
            d = (p >= 0 && p < cap) ? p : -1;
            wt = w[t * K + lane];
        }
        int dk[KM];
        float wk[KM];
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            dk[k] = __builtin_amdgcn_readlane(d, k);
            wk[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), k));
        }

        uint4 buf[KM][U];
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            if (dk[k] < 0) continue;
            const uint4* yr = y + (int64_t)dk[k] * nvec;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * kWave + lane;
                if (v < nvec) buf[k][u] = load_nt(yr + v);
            }
        }
        uint4* orow = out + t * nvec;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kWave + lane;
            if (v >= nvec) continue;
            float acc[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
            for (int k = 0; k < KM; ++k) {
                if (dk[k] < 0) continue;
                const uint4 q = buf[k][u];
                const float s = wk[k];
                acc[0] = __builtin_fmaf(s, bf16_lo(q.x), acc[0]);
                acc[1] = __builtin_fmaf(s, bf16_hi(q.x), acc[1]);
                acc[2] = __builtin_fmaf(s, bf16_lo(q.y), acc[2]);
                acc[3] = __builtin_fmaf(s, bf16_hi(q.y), acc[3]);
                acc[4] = __builtin_fmaf(s, bf16_lo(q.z), acc[4]);
                acc[5] = __builtin_fmaf(s, bf16_hi(q.z), acc[5]);
                acc[6] = __builtin_fmaf(s, bf16_lo(q.w), acc[6]);
                acc[7] = __builtin_fmaf(s, bf16_hi(q.w), acc[7]);
            }
            uint4 r;
            r.x = pack_bf16x2(acc[0], acc[1]);
            r.y = pack_bf16x2(acc[2], acc[3]);
            r.z = pack_bf16x2(acc[4], acc[5]);
            r.w = pack_bf16x2(acc[6], acc[7]);
            store_nt(orow + v, r);
        }
    }
}

hipError_t preload_combine() {
    hipFuncAttributes a;
    return hipFuncGetAttributes(&a, reinterpret_cast<const void*>(&combine_kernel<8, CGD_COMBINE_U>));
}

hipError_t launch_combine(const void* expert_out, int64_t cap, int H, const int32_t* dst_row, const float* w,
                          int64_t T, int K, void* out, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const uint4* yv = reinterpret_cast<const uint4*>(expert_out);
    uint4* ov = reinterpret_cast<uint4*>(out);
    const int nvec = H / 8;
    // token ranges within 32-bit work-item ids; the kernel indexes tokens
    // relative to the pointers it is given
#define CGD_COMBINE(KM, U)                                                                                          \
    do {                                                                                                            \
        const int nchunk = (nvec + U * kWave - 1) / (U * kWave);                                                    \
        const int64_t tper = tokens_per_launch(nchunk);                                                             \
        constexpr unsigned kLds = KM > 8 ? CGD_COMBINE_LDS_WIDE : CGD_COMBINE_LDS_CAP;                              \
        for (int64_t t0 = 0; t0 < T; t0 += tper) {                                                                  \
            const int64_t nt = T - t0 < tper ? T - t0 : tper;                                                       \
            const int64_t blocks = (nt * nchunk + kCombineWaves - 1) / kCombineWaves;                               \
            const dim3 grid((unsigned)blocks), block(kCombineWaves * kWave);                                        \
            hipLaunchKernelGGL((combine_kernel<KM, U>), grid, block, kLds, stream, yv, cap, nvec,                   \
                               nchunk, dst_row + t0 * K, w + t0 * K, nt, K, ov + t0 * nvec);                         \
        }                                                                                                           \
    } while (0)
    if (K <= 2)
        CGD_COMBINE(2, CGD_COMBINE_U);
    else if (K <= 4)
        CGD_COMBINE(4, CGD_COMBINE_U);
    else if (K <= 8)
        CGD_COMBINE(8, CGD_COMBINE_U);
    else
        CGD_COMBINE(16, CGD_COMBINE_U);
#undef CGD_COMBINE
    return hipGetLastError();
}

}  // namespace cgd
