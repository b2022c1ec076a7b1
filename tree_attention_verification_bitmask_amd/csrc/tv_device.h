// Device-side helpers shared by the HIP kernels of libtreeverify (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "treeverify.h"

namespace tv {

// Report a device-side error: (code << 24) | index, combined by atomic max so
// the final word does not depend on which thread got there first.
__device__ __forceinline__ void report(int32_t *err, int code, int64_t index) {
    if (err) atomicMax(err, (int32_t)((code << 24) | (int32_t)(index & 0xFFFFFF)));
}

// Checks a request's node range and returns N_b, or -1 if it is inconsistent.
__device__ __forceinline__ int request_nodes(const int32_t *cu_nodes, int b, int total_nodes,
                                             int max_nodes, int *lo_out) {
    const int lo = cu_nodes[b];
    const int hi = cu_nodes[b + 1];
    *lo_out = lo;
    if (lo < 0 || hi < lo || hi > total_nodes || hi - lo > max_nodes) return -1;
    return hi - lo;
}

// Request of node t: the b with cu_nodes[b] <= t < cu_nodes[b+1] (binary
// search), or -1 when the offsets do not place t in any request.
__device__ __forceinline__ int request_of(const int32_t *cu, int batch, int t) {
    int lo = 0, hi = batch;  // invariant: cu[lo] <= t < cu[hi] when t is inside
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= t) lo = mid;
        else hi = mid;
    }
    return (cu[lo] <= t && t < cu[lo + 1]) ? lo : -1;
}

// bf16 <-> fp32.  bf16 is stored as the upper half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16 pair (round to nearest even, hardware convert).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
    bf16x2_t v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace tv
