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

// Last-block-done handshake across the whole grid (blocks may sit on
// different XCDs, each with its own L2). Every thread publishes its global
// writes with a device-scope fence, then one thread takes a ticket; the block
// that takes the last ticket sees all other blocks' writes after its own
// acquire fence, and resets the ticket for the next launch.
__device__ __forceinline__ bool last_block_done(unsigned int* ticket) {
    __shared__ bool s_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned int prev = atomicAdd(ticket, 1u);
        s_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (s_last) __threadfence();
    return s_last;
}

__device__ __forceinline__ void reset_ticket(unsigned int* ticket) {
    if (threadIdx.x == 0) atomicExch(ticket, 0u);
}

}  // namespace cgd
