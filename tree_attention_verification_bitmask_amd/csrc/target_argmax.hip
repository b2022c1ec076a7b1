// tree_target_argmax: the target's greedy choice at every node.
//
// [TSD] = "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
// Tree Attention Accelerate LLM Serving" (llms.blog), section "Verification
// and Acceptance Algorithms", greedy tree verification: the target prediction
// at a node is the argmax of that node's logits.
//
// Pure streaming: every logit is read once, so HBM bandwidth bounds it.  One
// 1024-thread workgroup per row.  Each thread keeps kUnroll 16-byte loads in
// flight (128 KB per workgroup), visits its elements in increasing index
// order and keeps the first best; the workgroup then reduces 64-bit keys
// (order-preserving image of the value in the high half, the complement of
// the index in the low half) so the maximum key is the largest value at the
// lowest index.  NaN ranks above every number; -0 equals +0.
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {
namespace {

constexpr int kArgThreads = 1024;
constexpr int kArgWaves = kArgThreads / 64;
constexpr int kUnroll = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Key of (value, index): larger key = better candidate.
__device__ __forceinline__ uint64_t arg_key(float v, int idx) {
    uint32_t hi;
    if (v != v) {
        hi = 0xFFFFFFFFu;
    } else {
        if (v == 0.f) v = 0.f;  // -0 and +0 are one value
        const uint32_t u = __float_as_uint(v);
        hi = (u >> 31) ? ~u : (u | 0x80000000u);
    }
    return ((uint64_t)hi << 32) | (uint32_t)~(uint32_t)idx;
}

// v (at index i) beats the current best, seen at a lower index, only if it
// is the first element, strictly larger, or NaN over a number.
__device__ __forceinline__ void consider(float v, int i, float &best, int &bi) {
    if (bi < 0 || v > best || (v != v && best == best)) {
        best = v;
        bi = i;
    }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

template <bool BF16>
__global__ void __launch_bounds__(kArgThreads) target_argmax_kernel(const void *__restrict__ logits, int vocab,
                                                                     int32_t *__restrict__ token) {
    __shared__ uint64_t wbest[kArgWaves];
    constexpr int kEs = BF16 ? 2 : 4;
    constexpr int kPer = 16 / kEs;  // elements per 16-byte load
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const char *rbase = reinterpret_cast<const char *>(logits) + (int64_t)row * vocab * kEs;
    float best = -INFINITY;
    int bi = -1;
    // vector part: only when every row starts 16-byte aligned
    const bool vec = ((int64_t)vocab * kEs) % 16 == 0;
    const int nvec = vec ? vocab / kPer : 0;
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(rbase);
    constexpr int kStep = kArgThreads * kUnroll;
    for (int base = 0; base < nvec; base += kStep) {
        u32x4 buf[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int j = base + u * kArgThreads + tid;
            buf[u] = j < nvec ? __builtin_nontemporal_load(vp + j) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int j = base + u * kArgThreads + tid;
            if (j < nvec) {
                const uint32_t w[4] = {buf[u][0], buf[u][1], buf[u][2], buf[u][3]};
                if (BF16) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        consider(bf16_to_f32((uint16_t)(w[q] & 0xFFFF)), j * kPer + 2 * q, best, bi);
                        consider(bf16_to_f32((uint16_t)(w[q] >> 16)), j * kPer + 2 * q + 1, best, bi);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) consider(__uint_as_float(w[q]), j * kPer + q, best, bi);
                }
            }
        }
    }
    // scalar tail (and every element when rows are not 16-byte aligned)
    for (int i = nvec * kPer + tid; i < vocab; i += kArgThreads) {
        const float v = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(rbase)[i])
                             : reinterpret_cast<const float *>(rbase)[i];
        consider(v, i, best, bi);
    }
    // Threads that saw nothing hold index -1 and the lowest key.
    uint64_t key = bi < 0 ? 0ull : arg_key(best, bi);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = ((uint64_t)(uint32_t)__shfl_xor((int)(key >> 32), off, 64) << 32) |
                           (uint32_t)__shfl_xor((int)(uint32_t)key, off, 64);
        key = o > key ? o : key;
    }
    if ((tid & 63) == 0) wbest[tid >> 6] = key;
    __syncthreads();
    if (tid == 0) {
        uint64_t k = wbest[0];
#pragma unroll
        for (int w = 1; w < kArgWaves; ++w) k = wbest[w] > k ? wbest[w] : k;
        token[row] = (int32_t)~(uint32_t)k;
    }
}

}  // namespace

hipError_t launch_target_argmax(const void *logits, int rows, int vocab, tv_dtype dtype, int32_t *token,
                                hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    if (dtype == TV_BF16)
        hipLaunchKernelGGL(target_argmax_kernel<true>, dim3(rows), dim3(kArgThreads), 0, stream, logits, vocab,
                           token);
    else
        hipLaunchKernelGGL(target_argmax_kernel<false>, dim3(rows), dim3(kArgThreads), 0, stream, logits, vocab,
                           token);
    return hipGetLastError();
}

}  // namespace tv
