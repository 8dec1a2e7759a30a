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

// Copy n (<= ITEMS * blockDim.x) routing entries of one tile into LDS as
// int32, entries outside [0, E) becoming -1. All global loads of a thread are
// issued before any LDS store, so the tile costs one memory round trip.
template <int ITEMS>
__device__ __forceinline__ void stage_routing(const int64_t* __restrict__ src, int n, int E, int32_t* dst) {
    int64_t v[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int i = threadIdx.x + j * blockDim.x;
        v[j] = (i < n) ? src[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int i = threadIdx.x + j * blockDim.x;
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

__device__ __forceinline__ void reset_ticket(unsigned int* ticket) {
    if (threadIdx.x == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace cgd
