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
#include "path_walk.h"
#include "tv_launch.h"

namespace tv {
namespace {

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
    int pk[kWalkPerLane];
    int dk[kWalkPerLane];
    walk_load(par, dr, tg, n, pk, dk, stg);
    __syncthreads();
    int next;
    const int len = walk_registers(pk, dk, stg, n, root_want, max_depth, idx, &next);
    if (lane == 0) {
        accept_len[b] = len;
        next_token[b] = next;
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
