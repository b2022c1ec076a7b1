// tree_mask_build: packed ancestor-or-self mask, levels and position ids.
//
// [TSD] = "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
// Tree Attention Accelerate LLM Serving" (llms.blog), section "The Tree
// Attention Mechanism", parts 2 ("2D Causal Tree Mask") and 3 ("Tree
// Positional IDs").
//
// One workgroup per request.  The request's parent array (at most
// TV_MAX_NODES entries) is first copied to LDS in one coalesced pass, so the
// walks below cost LDS latency per step instead of a global-memory round
// trip.  Then one thread per node walks its parent pointers toward the root.
// Because a valid parent index is always smaller than its child's, the walk
// visits strictly decreasing indices, so the packed row can be streamed out
// from its highest word to its lowest with one 64-bit accumulator: a word is
// written as soon as the walk drops below it, and every word is written
// exactly once.  The walk is bounded by max_depth steps; every parent is
// range-checked before it is followed, so a bad tree cannot send a thread out
// of bounds.
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {
namespace {

constexpr int kMaskThreads = 256;

__global__ void __launch_bounds__(kMaskThreads) mask_build_kernel(
    const int32_t *__restrict__ parent, const int32_t *__restrict__ cu_nodes,
    const int32_t *__restrict__ prefix_len, int total_nodes, int max_nodes, int max_depth, int words,
    uint64_t *__restrict__ anc, int32_t *__restrict__ level, int32_t *__restrict__ pos,
    int32_t *__restrict__ err) {
    __shared__ int32_t spar[TV_MAX_NODES];
    const int b = blockIdx.x;
    int lo;
    const int n = request_nodes(cu_nodes, b, total_nodes, max_nodes, &lo);
    const int P = prefix_len[b];
    if ((n < 0) | (P < 0)) {  // (no short-circuit: both reads in flight together)
        if (threadIdx.x == 0) report(err, TV_DEVERR_BAD_REQUEST, b);
        return;
    }
    const int32_t *par = parent + lo;
    // every load first, then the LDS stores (a store right after its load
    // would wait for it: one memory round trip per 256 nodes)
    constexpr int kPer = (TV_MAX_NODES + kMaskThreads - 1) / kMaskThreads;
    int pv[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int i = threadIdx.x + r * kMaskThreads;
        pv[r] = i < n ? par[i] : 0;
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int i = threadIdx.x + r * kMaskThreads;
        if (i < n) spar[i] = pv[r];
    }
    __syncthreads();

    for (int i = threadIdx.x; i < n; i += kMaskThreads) {
        const int64_t t = (int64_t)lo + i;
        uint64_t *row = anc + t * words;
        int cw = words - 1;  // highest word not yet written
        uint64_t acc = 0;
        int lev = 0;
        int v = i;
        bool bad = false;
        while (true) {
            ++lev;
            if (lev > max_depth) {
                report(err, TV_DEVERR_TOO_DEEP, t);
                bad = true;
                break;
            }
            const int vw = v >> 6;
            while (cw > vw) {
                row[cw--] = acc;
                acc = 0;
            }
            acc |= 1ull << (v & 63);
            const int p = spar[v];
            if (p < -1 || p >= v) {
                report(err, TV_DEVERR_BAD_PARENT, (int64_t)lo + v);
                bad = true;
                break;
            }
            if (p < 0) break;
            v = p;
        }
        if (bad) {
            for (int w = 0; w < words; ++w) row[w] = 0;
            level[t] = 0;
            pos[t] = 0;
            continue;
        }
        while (cw >= 0) {
            row[cw--] = acc;
            acc = 0;
        }
        level[t] = lev;
        pos[t] = P + lev - 1;
    }
}

}  // namespace

hipError_t launch_mask_build(const int32_t *parent, const int32_t *cu_nodes, const int32_t *prefix_len,
                             int batch, int total_nodes, int max_nodes, int max_depth, uint64_t *anc,
                             int32_t *level, int32_t *pos, int32_t *err, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    const int words = (max_nodes + 63) / 64;
    hipLaunchKernelGGL(mask_build_kernel, dim3(batch), dim3(kMaskThreads), 0, stream, parent, cu_nodes,
                       prefix_len, total_nodes, max_nodes, max_depth, words, anc, level, pos, err);
    return hipGetLastError();
}

}  // namespace tv
