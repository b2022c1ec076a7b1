// tree_accept_greedy: the temperature-0 acceptance walk.
//
// [TSD] = "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
// Tree Attention Accelerate LLM Serving" (llms.blog), section "Verification
// and Acceptance Algorithms", greedy tree verification.
//
// One wavefront per request.  Each step looks for the current node's child
// carrying the token the target chose at the current node: the 64 lanes test
// 64 candidate nodes at a time (parent == current && draft == wanted token)
// and a ballot picks the lowest matching index.  The walk is at most
// max_depth steps of at most ceil(N/64) ballots each.  Every lane follows the
// same (uniform) path, so lane 0 alone writes the outputs.
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {
namespace {

__global__ void __launch_bounds__(64) accept_greedy_kernel(
    const int32_t *__restrict__ parent, const int32_t *__restrict__ draft,
    const int32_t *__restrict__ target, const int32_t *__restrict__ root_target,
    const int32_t *__restrict__ cu_nodes, int total_nodes, int max_depth,
    int32_t *__restrict__ accept_len, int32_t *__restrict__ accept_idx,
    int32_t *__restrict__ next_token, int32_t *__restrict__ err) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    int lo;
    // the walk needs no per-request node cap: pass total_nodes as the cap
    const int n = request_nodes(cu_nodes, b, total_nodes, total_nodes, &lo);
    int32_t *idx = accept_idx + (int64_t)b * max_depth;
    if (n < 0) {
        if (lane == 0) report(err, TV_DEVERR_BAD_REQUEST, b);
        return;
    }
    const int32_t *par = parent + lo;
    const int32_t *dr = draft + lo;
    const int32_t *tg = target + lo;

    int want = root_target[b];
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
        accept_len[b] = len;
        next_token[b] = want;
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
