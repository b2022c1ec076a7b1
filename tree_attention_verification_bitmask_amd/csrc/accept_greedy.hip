// tree_accept_greedy: the temperature-0 acceptance walk.
//
// [TSD] = "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
// Tree Attention Accelerate LLM Serving" (llms.blog), section "Verification
// and Acceptance Algorithms", greedy tree verification.
//
// One wavefront per request.  A node is acceptable when its draft token is
// the token the target chose at its parent (the root's choice for a node
// under the implicit root) and is not a dead leaf (negative token).  That
// test depends only on the node, so it is done for every node at once: lane
// l holds nodes l, l + 64, ... with their parent index and acceptability bit
// in registers.  The walk then needs no memory: each step finds the current
// node's lowest-index acceptable child with one ballot per 64 nodes.  The
// target tokens are staged in LDS for the acceptability test and the final
// next token.  A request above TV_MAX_NODES nodes (the call takes no node
// cap) falls back to testing candidates from global memory at each step.
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {
namespace {

constexpr int kPerLane = (TV_MAX_NODES + 63) / 64;  // nodes held per lane

// The same walk for a request too large to hold in registers: each step
// tests the candidates (parent == current, draft == wanted token) 64 at a
// time from global memory and a ballot picks the lowest matching index.
__device__ void walk_global(const int32_t *par, const int32_t *dr, const int32_t *tg, int n,
                            int want, int max_depth, int32_t *idx, int32_t *len_out,
                            int32_t *next_out) {
    const int lane = threadIdx.x;
    int cur = -1;
    int len = 0;
    while (len < max_depth) {
        int found = -1;
        for (int base = 0; base < n; base += 64) {
            const int j = base + lane;
            bool m = false;
            if (j < n) {
                const int dj = dr[j];
                m = (par[j] == cur) && (dj >= 0) && (dj == want);
            }
            const unsigned long long bal = __ballot(m);
            if (bal) {
                found = base + __builtin_ctzll(bal);
                break;
            }
        }
        if (found < 0) break;
        if (lane == 0) idx[len] = found;
        ++len;
        cur = found;
        want = tg[found];
    }
    for (int j = len + lane; j < max_depth; j += 64) idx[j] = -1;
    if (lane == 0) {
        *len_out = len;
        *next_out = want;
    }
}

__global__ void __launch_bounds__(64) accept_greedy_kernel(
    const int32_t *__restrict__ parent, const int32_t *__restrict__ draft,
    const int32_t *__restrict__ target, const int32_t *__restrict__ root_target,
    const int32_t *__restrict__ cu_nodes, int total_nodes, int max_depth,
    int32_t *__restrict__ accept_len, int32_t *__restrict__ accept_idx,
    int32_t *__restrict__ next_token, int32_t *__restrict__ err) {
    __shared__ int32_t stg[TV_MAX_NODES];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    int lo;
    // the walk needs no per-request node cap: pass total_nodes as the cap
    const int n = request_nodes(cu_nodes, b, total_nodes, total_nodes, &lo);
    const int root_want = root_target[b];  // (read alongside the offsets)
    int32_t *idx = accept_idx + (int64_t)b * max_depth;
    if (n < 0) {
        if (lane == 0) report(err, TV_DEVERR_BAD_REQUEST, b);
        return;
    }
    const int32_t *par = parent + lo;
    const int32_t *dr = draft + lo;
    const int32_t *tg = target + lo;
    if (n > TV_MAX_NODES) {
        // too many nodes to hold: test the children straight from memory
        walk_global(par, dr, tg, n, root_want, max_depth, idx, accept_len + b, next_token + b);
        return;
    }
    const int nk = (n + 63) / 64;  // wave-uniform

    int pk[kPerLane];
    int dk[kPerLane];
    int tk[kPerLane];
    // every load first, then the LDS stores: a store right after its load
    // would wait for it, one memory round trip per 64 nodes
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
        const int j = 64 * k + lane;
        pk[k] = -2;
        dk[k] = -1;
        tk[k] = 0;
        if (k < nk && j < n) {
            pk[k] = par[j];
            dk[k] = dr[j];
            tk[k] = tg[j];
        }
    }
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
        const int j = 64 * k + lane;
        if (k < nk && j < n) stg[j] = tk[k];
    }
    __syncthreads();
    // acceptable[j]: draft[j] == the target's choice at parent[j]
    uint32_t okbits = 0;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
        if (k < nk) {
            const int p = pk[k];
            const int want = p == -1 ? root_want : (p >= 0 && p < n ? stg[p] : -1);
            if (dk[k] >= 0 && dk[k] == want) okbits |= 1u << k;
        }
    }

    int cur = -1;
    int len = 0;
    while (len < max_depth) {
        int found = -1;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            if (k >= nk) break;
            const unsigned long long bal = __ballot(((okbits >> k) & 1u) && pk[k] == cur);
            if (bal) {
                found = 64 * k + __builtin_ctzll(bal);
                break;
            }
        }
        if (found < 0) break;
        if (lane == 0) idx[len] = found;
        ++len;
        cur = found;
    }
    for (int j = len + lane; j < max_depth; j += 64) idx[j] = -1;
    if (lane == 0) {
        accept_len[b] = len;
        next_token[b] = cur < 0 ? root_want : stg[cur];
    }
}

}  // namespace

hipError_t launch_accept_greedy(const int32_t *parent, const int32_t *draft, const int32_t *target,
                                const int32_t *root_target, const int32_t *cu_nodes, int batch,
                                int total_nodes, int max_depth, int32_t *accept_len, int32_t *accept_idx,
                                int32_t *next_token, int32_t *err, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    hipLaunchKernelGGL(accept_greedy_kernel, dim3(batch), dim3(64), 0, stream, parent, draft, target,
                       root_target, cu_nodes, total_nodes, max_depth, accept_len, accept_idx,
                       next_token, err);
    return hipGetLastError();
}

}  // namespace tv
