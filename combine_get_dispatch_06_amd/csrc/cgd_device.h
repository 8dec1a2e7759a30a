// Device helpers shared by the gfx950 kernels of libcgd.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cgd_launch.h"

namespace cgd {

constexpr int kWave = 64;  // CDNA wavefront width

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// bf16 <-> fp32 on packed pairs. A 32-bit word holds element 2i in its low
// half and element 2i+1 in its high half (little-endian storage order).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 pair, round to nearest even (gfx950 has a
// native packed conversion for this; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    float2_t f = {lo, hi};
    bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

// ---- FP8 (OCP e4m3fn) payload -------------------------------------------
// One scale per token and block of 128 channels (kFp8Block). Scale formats:
// 0 fp32 amax/448; 1 fp32 power of two (the smallest 2^k >= amax/448);
// 2 that power of two as the byte k + 127 (UE8M0). Every step is fp32, with
// correctly rounded division, so the 8-bit codes are decided exactly as the
// format's definition states.
constexpr int kFp8Block = 128;
constexpr float kE4m3Max = 448.0f;  // largest finite e4m3fn value

struct Fp8Scale {
    float mul;      // multiplier applied before encoding
    float scale;    // dequantisation scale (fp32 formats)
    uint32_t ue8m0; // biased exponent byte (format 2)
};

__device__ __forceinline__ Fp8Scale fp8_block_scale(float amax, int fmt) {
    amax = amax < 1e-4f ? 1e-4f : amax;  // a block of zeros keeps a positive scale
    Fp8Scale r;
    if (fmt == 0) {
        r.mul = kE4m3Max / amax;
        r.scale = amax / kE4m3Max;
        r.ue8m0 = 0;
    } else {
        int e;
        const float m = frexpf(amax / kE4m3Max, &e);
        const int k = (m == 0.5f) ? e - 1 : e;
        r.mul = ldexpf(1.0f, -k);
        r.scale = ldexpf(1.0f, k);
        r.ue8m0 = (uint32_t)(k + 127);
    }
    return r;
}

// Max over the 16 lanes of an aligned lane group (one 128-channel block when
// each lane holds 8 channels).
__device__ __forceinline__ float group16_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 8, kWave));
    v = fmaxf(v, __shfl_xor(v, 4, kWave));
    v = fmaxf(v, __shfl_xor(v, 2, kWave));
    v = fmaxf(v, __shfl_xor(v, 1, kWave));
    return v;
}

// Max over the 8 lanes of an aligned lane group (one 128-channel block when
// each lane holds 16 channels).
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 4, kWave));
    v = fmaxf(v, __shfl_xor(v, 2, kWave));
    v = fmaxf(v, __shfl_xor(v, 1, kWave));
    return v;
}

__device__ __forceinline__ float clamp_e4m3(float v) {
    v = v > kE4m3Max ? kE4m3Max : v;  // NaN passes through unchanged
    return v < -kE4m3Max ? -kE4m3Max : v;
}

// Four fp32 values -> four e4m3fn bytes (element 0 in the low byte). gfx950's
// conversion rounds to nearest even but does not saturate, hence the clamp.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a), clamp_e4m3(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(c), clamp_e4m3(d), w, true);
    return (uint32_t)w;
}

// Absolute max of the 8 bf16 values of a 16-byte vector.
__device__ __forceinline__ float absmax_bf16x8(const uint4& q) {
    float m = fmaxf(fabsf(bf16_lo(q.x)), fabsf(bf16_hi(q.x)));
    m = fmaxf(m, fmaxf(fabsf(bf16_lo(q.y)), fabsf(bf16_hi(q.y))));
    m = fmaxf(m, fmaxf(fabsf(bf16_lo(q.z)), fabsf(bf16_hi(q.z))));
    return fmaxf(m, fmaxf(fabsf(bf16_lo(q.w)), fabsf(bf16_hi(q.w))));
}

// 8 bf16 values times mul -> 8 e4m3fn bytes.
__device__ __forceinline__ uint2 quantize_bf16x8(const uint4& q, float mul) {
    uint2 r;
    r.x = pack_e4m3x4(bf16_lo(q.x) * mul, bf16_hi(q.x) * mul, bf16_lo(q.y) * mul, bf16_hi(q.y) * mul);
    r.y = pack_e4m3x4(bf16_lo(q.z) * mul, bf16_hi(q.z) * mul, bf16_lo(q.w) * mul, bf16_hi(q.w) * mul);
    return r;
}

// 16 bf16 values (two 16-byte vectors) times mul -> 16 e4m3fn bytes.
__device__ __forceinline__ uint4 quantize_bf16x16(const uint4& a, const uint4& b, float mul) {
    const uint2 lo = quantize_bf16x8(a, mul), hi = quantize_bf16x8(b, mul);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Streaming 16-byte global accesses: data touched once should not displace
// reusable lines in L2 / MALL.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
    uint4 v;
    v.x = __builtin_nontemporal_load(&p->x);
    v.y = __builtin_nontemporal_load(&p->y);
    v.z = __builtin_nontemporal_load(&p->z);
    v.w = __builtin_nontemporal_load(&p->w);
    return v;
}

__device__ __forceinline__ void store_nt(uint4* p, const uint4& v) {
    __builtin_nontemporal_store(v.x, &p->x);
    __builtin_nontemporal_store(v.y, &p->y);
    __builtin_nontemporal_store(v.z, &p->z);
    __builtin_nontemporal_store(v.w, &p->w);
}

__device__ __forceinline__ uint2 load_nt(const uint2* p) {
    uint2 v;
    v.x = __builtin_nontemporal_load(&p->x);
    v.y = __builtin_nontemporal_load(&p->y);
    return v;
}

__device__ __forceinline__ void store_nt(uint2* p, const uint2& v) {
    __builtin_nontemporal_store(v.x, &p->x);
    __builtin_nontemporal_store(v.y, &p->y);
}

// Optional per-row side payload moved with dispatched rows (the FP8 scales):
// nsb elements of sbytes (4 or 1) bytes per token at src + t*st + j*sb
// (element strides, so column-major scales work too), copied to
// dst[row * nsb + j].
struct SideRows {
    const void* src;
    int64_t st, sb;
    int nsb;
    int sbytes;
    void* dst;
};

// Copy token t's side payload to receive row `row` (lanes stride the elements).
__device__ __forceinline__ void copy_side_row(const SideRows& s, int64_t t, int64_t row, int lane) {
    for (int j = lane; j < s.nsb; j += kWave) {
        const int64_t i = t * s.st + (int64_t)j * s.sb;
        if (s.sbytes == 4)
            static_cast<float*>(s.dst)[row * s.nsb + j] = static_cast<const float*>(s.src)[i];
        else
            static_cast<uint8_t*>(s.dst)[row * s.nsb + j] = static_cast<const uint8_t*>(s.src)[i];
    }
}

// Up to this top-k, a kernel with one token per thread loads its token's
// routing straight into registers (the K loads of a wave together use every
// byte of the lines they touch) instead of staging the tile through LDS:
// get_dispatch_layout alone measured 4.81 against 5.27 us at prefill and
// 6.23 against 6.64 Zipf-skewed; at top-16 the staged form is faster (11.9
// against 12.5 us).
#ifndef CGD_DIRECT_TOPK
#define CGD_DIRECT_TOPK 8
#endif
constexpr int kDirectTopk = CGD_DIRECT_TOPK;

// Copy n (<= ITEMS * BLOCK) routing entries of one tile into LDS as int32,
// entries outside [0, E) becoming -1, with a block of BLOCK threads. All
// global loads of a thread are issued before any LDS store, so the tile costs
// one memory round trip. Block sizes are compile-time constants throughout:
// blockDim.x would be a vector load from the kernel-argument segment at the
// start of every wave.
template <int ITEMS, int BLOCK>
__device__ __forceinline__ void stage_routing(const int64_t* __restrict__ src, int n, int E, int32_t* dst) {
    int64_t v[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int i = threadIdx.x + j * BLOCK;
        v[j] = (i < n) ? src[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int i = threadIdx.x + j * BLOCK;
        if (i < n) dst[i] = (v[j] >= 0 && v[j] < E) ? (int32_t)v[j] : -1;
    }
}

// Cross-block synchronisation. Blocks of one grid may sit on different XCDs,
// each with its own L2. On gfx950 a device-scope release writes back the XCD's
// L2 and a device-scope acquire invalidates it, so each is issued once per
// block by thread 0, ordered with the block's other waves by a barrier. A
// workgroup barrier does not wait for a wave's outstanding vector stores, and
// thread 0's release waits only for its own wave's, so every wave first waits
// until its stores are acknowledged by L2; thread 0 then waits for the L2
// write-back itself before taking the ticket. These waits are explicit
// (s_waitcnt with all counters 0), which the compiler keeps as written.

// Last-block-done handshake among `nblocks` blocks: each block publishes its
// writes and takes a ticket; the block that takes the last ticket acquires
// every other block's writes and must reset the ticket (reset_ticket).
__device__ __forceinline__ bool last_block_done(unsigned int* ticket, unsigned int nblocks) {
    __shared__ bool s_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __builtin_amdgcn_s_waitcnt(0);
        const unsigned int prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == nblocks - 1);
        if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    return s_last;
}

__device__ __forceinline__ bool last_block_done(unsigned int* ticket) { return last_block_done(ticket, gridDim.x); }

// ---- Per-tile layout work (shared by the layout kernel and the fused
// layout + dispatch plan): one token per thread, RW 64-bit words of rank mask
// per token (1 for R <= 64, 6 for R <= 384).

// Bitmask of the ranks the token's selected experts live on (e[k] < 0: none).
// lshift >= 0: L = 2^lshift experts per rank, the rank is a shift; else the
// expert -> rank table in LDS.
// Straight-line code: the ranks of all slots first (the table reads, at a
// valid index for every slot, all in flight together), then selects; a
// branch per slot around a table read costs a wait per slot.
template <int RW>
__device__ __forceinline__ void token_rank_mask(const int (&e)[kMaxTopk], const int16_t* s_rank_of, int lshift,
                                                uint64_t (&m)[RW]) {
    int r[kMaxTopk];
    if (lshift >= 0) {
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k) r[k] = e[k] >> lshift;
    } else {
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k) r[k] = s_rank_of[max(e[k], 0)];
    }
#pragma unroll
    for (int w = 0; w < RW; ++w) m[w] = 0;
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
#pragma unroll
        for (int w = 0; w < RW; ++w)
            m[w] |= (e[k] >= 0 && (r[k] >> 6) == w) ? 1ull << (r[k] & 63) : 0ull;
    }
}

// Distinct tokens per rank, added to s_rank (LDS, [R]): one ballot per rank
// over the wave's tokens, lane (r % 64) adds the popcount for rank r. Also
// stores the thread's mask in s_mask[tid * RW + w]. s_bal (optional, LDS
// [waves, R]) receives each rank's ballot: the wave's group word of the
// rank-granular dispatch plan.
template <int RW>
__device__ __forceinline__ void count_rank_tokens(const uint64_t (&m)[RW], int R, int32_t* s_rank, uint64_t* s_mask,
                                                  uint64_t* s_bal = nullptr) {
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int w = 0; w < RW; ++w) {
        const int rbeg = w * kWave;
        const int rend = min(R, rbeg + kWave);
        int cnt = 0;
        for (int r = rbeg; r < rend; ++r) {
            const uint64_t b = ballot((m[w] >> (r & 63)) & 1ull);
            if (lane == (r & 63)) cnt = __popcll(b);
            if (s_bal && lane == 0) s_bal[wave * R + r] = b;
        }
        if (rbeg + lane < rend && cnt) atomicAdd(&s_rank[rbeg + lane], cnt);
        s_mask[threadIdx.x * RW + w] = m[w];
    }
}

// Four rank flags (bits 0..3 of b) as four 0/1 bytes of a little-endian word:
// the multiplier puts bit i at bit 8i, the mask keeps those bits.
__device__ __forceinline__ uint32_t flag_bytes4(uint32_t b) { return ((b & 0xFu) * 0x00204081u) & 0x01010101u; }

// The tile's is_token_in_rank rows (nt tokens, a contiguous byte range
// starting at out, 16-byte aligned). R % 4 == 0, R = 1 or R = 2: each thread
// stores its own token's row from its mask m (the widest aligned stores);
// other R: 16 bytes per store across token boundaries from the masks in
// s_mask (call after a barrier that follows count_rank_tokens).
template <int RW, int BLOCK>
__device__ __forceinline__ void store_token_in_rank(const uint64_t (&m)[RW], const uint64_t* s_mask, int nt, int R,
                                                    uint8_t* out) {
    if (R % 4 == 0 || R <= 2) {
        const int t = threadIdx.x;
        if (t >= nt) return;
        uint8_t* row = out + t * R;
        auto bits4 = [&](int p) {  // flags of ranks p..p+3 (p % 4 == 0: never straddles a word)
            uint64_t w = 0;
#pragma unroll
            for (int i = 0; i < RW; ++i)
                if ((p >> 6) == i) w = m[i];
            return flag_bytes4((uint32_t)(w >> (p & 63)));
        };
        if (R % 16 == 0) {
            for (int p = 0; p < R; p += 16)
                *reinterpret_cast<uint4*>(row + p) = make_uint4(bits4(p), bits4(p + 4), bits4(p + 8), bits4(p + 12));
        } else if (R % 8 == 0) {
            for (int p = 0; p < R; p += 8) *reinterpret_cast<uint2*>(row + p) = make_uint2(bits4(p), bits4(p + 4));
        } else if (R % 4 == 0) {
            for (int p = 0; p < R; p += 4) *reinterpret_cast<uint32_t*>(row + p) = bits4(p);
        } else if (R == 2) {
            *reinterpret_cast<uint16_t*>(row) = (uint16_t)bits4(0);
        } else {
            row[0] = (uint8_t)bits4(0);
        }
        return;
    }
    const int nbytes = nt * R;  // <= 256 * 384
    for (int c = threadIdx.x; c * 16 < nbytes; c += BLOCK) {
        const int b0 = c * 16;
        int tok = b0 / R;
        int r = b0 - tok * R;
        const int nb = min(16, nbytes - b0);
        uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j < nb) {
                const uint32_t bit = (uint32_t)(s_mask[tok * RW + (r >> 6)] >> (r & 63)) & 1u;
                wd[j >> 2] |= bit << ((j & 3) * 8);
            }
            if (++r == R) {
                r = 0;
                ++tok;
            }
        }
        if (nb == 16) {
            *reinterpret_cast<uint4*>(out + b0) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        } else {
            for (int j = 0; j < nb; ++j) out[b0 + j] = (uint8_t)(wd[j >> 2] >> ((j & 3) * 8));
        }
    }
}

// Exclusive prefix sum of n <= 2 * kRankTile integers v(0..n-1) by a block
// of kRankTile threads: out[i] = v(0) + ... + v(i-1) for i <= n (out[n] is the
// total). Thread i owns entries 2i and 2i+1; a wavefront scan with shuffles
// and one LDS word per wave combine them. v is evaluated once per entry.
template <class F>
__device__ __forceinline__ void block_exclusive_scan2(int n, F v, int32_t* out, int32_t* s_wsum) {
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int i0 = 2 * tid, i1 = 2 * tid + 1;
    const int c0 = (i0 < n) ? v(i0) : 0;
    const int c1 = (i1 < n) ? v(i1) : 0;
    const int own = c0 + c1;
    int inc = own;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int u = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += u;
    }
    if (lane == kWave - 1) s_wsum[wave] = inc;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_wsum[w];
    const int excl = before + inc - own;
    if (i0 < n) out[i0] = excl;
    if (i1 < n) out[i1] = excl + c0;
    if (tid == kRankTile - 1) out[n] = before + inc;  // entries >= n add 0
}

// Blocks of a plan past its tiles pull x toward the caches (L2, Infinity
// Cache) while the plan runs, so that the row copy that follows finds it
// there: the plan is latency-bound on a few CUs and leaves the others and
// the memory bandwidth idle, while a row copy reading x from HBM is bound by
// that latency. Each thread reads vectors b*BLOCK + tid + j*stride with
// ordinary loads, kInFlight at a time, and discards them.
#ifndef CGD_PREFETCH_BLOCKS
#define CGD_PREFETCH_BLOCKS 240
#endif
#ifndef CGD_PREFETCH_IN_FLIGHT
#define CGD_PREFETCH_IN_FLIGHT 8
#endif
constexpr int kPrefetchBlocks = CGD_PREFETCH_BLOCKS;

template <int BLOCK>
__device__ __forceinline__ void prefetch_rows(const uint4* __restrict__ p, int64_t n, int b, int nb) {
    constexpr int kInFlight = CGD_PREFETCH_IN_FLIGHT;
    const int64_t stride = (int64_t)nb * BLOCK;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)b * BLOCK + threadIdx.x; i < n; i += stride * kInFlight) {
        uint4 v[kInFlight];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) v[j] = (i + j * stride < n) ? p[i + j * stride] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    asm volatile("" ::"v"(acc));  // the loaded values are used, so the loads stay
}

// Blocks of a plan past its tiles that cast x to FP8 while the plan runs
// (the rank-granular dispatch with the cast): the (token, 1024-channel chunk)
// items of x, kCastInFlight per wave at a time, each lane 16 channels (two
// 16-byte bf16 vectors in, one 16-byte code vector out), an 8-lane group one
// 128-channel block, exactly as the per-token cast: codes q [T, H] and
// row-major scales [T, H/128] (fp32, or one UE8M0 byte for fmt 2). b, nb:
// this block among the nb casting blocks of BLOCK threads.
#ifndef CGD_CAST_IN_FLIGHT
#define CGD_CAST_IN_FLIGHT 2
#endif
constexpr int kCastInFlight = CGD_CAST_IN_FLIGHT;
template <int BLOCK>
__device__ __forceinline__ void cast_rows(const uint4* __restrict__ x, int64_t T, int H, int fmt,
                                          uint4* __restrict__ q, void* __restrict__ scales, int b, int nb) {
    const int nlv = H / 16;                  // lane vectors (16 channels) per row
    const int nchunk = (nlv + kWave - 1) / kWave;
    const int nsb = H / kFp8Block;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t waves = (int64_t)nb * (BLOCK / kWave);
    const int64_t w0 = (int64_t)b * (BLOCK / kWave) + (int)(threadIdx.x / kWave);
    const int64_t items = T * nchunk;
    for (int64_t i0 = w0; i0 < items; i0 += waves * kCastInFlight) {
        uint4 a[kCastInFlight], c[kCastInFlight];
        int64_t t[kCastInFlight];
        int v[kCastInFlight];
        bool in[kCastInFlight];
#pragma unroll
        for (int j = 0; j < kCastInFlight; ++j) {  // every item's loads first
            const int64_t it = i0 + j * waves;
            t[j] = it / nchunk;
            v[j] = (int)(it - t[j] * nchunk) * kWave + lane;
            in[j] = it < items && v[j] < nlv;  // whole 8-lane groups are in or out (nlv % 8 == 0)
            a[j] = c[j] = make_uint4(0, 0, 0, 0);
            if (in[j]) {
                const uint4* xr = x + (t[j] * nlv + v[j]) * 2;
                a[j] = xr[0];
                c[j] = xr[1];
            }
        }
#pragma unroll
        for (int j = 0; j < kCastInFlight; ++j) {
            const float m = in[j] ? fmaxf(absmax_bf16x8(a[j]), absmax_bf16x8(c[j])) : 0.0f;
            const Fp8Scale sc = fp8_block_scale(group8_max(m), fmt);
            if (!in[j]) continue;
            q[t[j] * nlv + v[j]] = quantize_bf16x16(a[j], c[j], sc.mul);
            if ((lane & 7) == 0) {
                const int64_t si = t[j] * nsb + v[j] / 8;
                if (fmt == 2)
                    static_cast<uint8_t*>(scales)[si] = (uint8_t)sc.ue8m0;
                else
                    static_cast<float*>(scales)[si] = sc.scale;
            }
        }
    }
}

__device__ __forceinline__ void reset_ticket(unsigned int* ticket) {
    if (threadIdx.x == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace cgd
