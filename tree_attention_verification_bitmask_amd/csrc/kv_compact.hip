// kv_compact_path: gather the accepted path's K/V rows into place; and
// tree_accept_commit: the acceptance walk and that gather in one launch.
//
// [TSD] = "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
// Tree Attention Accelerate LLM Serving" (llms.blog), section "KV Cache
// Rollback".
//
// One workgroup per (request, KV head).  The destination rows P+j and the
// source rows P+idx[j] overlap (a path [0, 2, 5] reads row P+2 and also
// writes it), so the workgroup first reads every source row of its head
// slice into LDS, waits on a barrier, and only then writes.  Different KV heads touch disjoint bytes, so
// workgroups never race.  Rows already in place (idx[j] == j) are skipped.
// The path indices are loaded once, one per thread, checked together (one
// barrier-wide OR), and shared through LDS.
#include "path_walk.h"
#include "tv_launch.h"

namespace tv {
namespace {

constexpr int kCompactThreads = 256;
static_assert(TV_MAX_DEPTH <= kCompactThreads, "one path entry per thread");

// ROW_BYTES = head_dim * element size: 128, 256 or 512 bytes.
template <int ROW_BYTES>
__global__ void __launch_bounds__(kCompactThreads) kv_compact_kernel(
    uint8_t *__restrict__ kc, uint8_t *__restrict__ vc, const int32_t *__restrict__ cu_nodes,
    const int32_t *__restrict__ kv_start, const int32_t *__restrict__ prefix_len,
    const int32_t *__restrict__ accept_len, const int32_t *__restrict__ accept_idx, int total_nodes,
    int max_depth, int64_t kv_rows, int hkv, int32_t *__restrict__ new_len, int32_t *__restrict__ err) {
    extern __shared__ uint4 stage[];                                       // [2][max_depth][V16]
    __shared__ int32_t sidx[TV_MAX_DEPTH];
    const int b = blockIdx.x;
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    int lo;
    const int n = request_nodes(cu_nodes, b, total_nodes, total_nodes, &lo);
    const int P = prefix_len[b];
    const int64_t ks = kv_start[b];
    const int L = accept_len[b];
    // The path row is read before the sizes are checked (it lies in bounds
    // whatever they are), and the checks use no short-circuit, so all these
    // reads are in flight together instead of one round trip each.
    const int s_raw = tid < max_depth ? accept_idx[(int64_t)b * max_depth + tid] : 0;
    // L > n is rejected too: a path through n nodes is at most n long, and the
    // gather writes rows P .. P + L - 1, which must stay inside the request.
    if ((n < 0) | (P < 0) | (ks < 0) | (ks + P + n > kv_rows) | (L < 0) | (L > max_depth) | (L > n)) {
        if (g == 0 && tid == 0) report(err, TV_DEVERR_BAD_REQUEST, b);
        return;
    }
    const int s = tid < L ? s_raw : 0;
    const bool bad = tid < L && (s < 0 || s >= n);
    if (tid < L) sidx[tid] = s;
    if (__syncthreads_or(bad)) {  // uniform: every thread sees the same OR
        if (g == 0 && tid == 0) report(err, TV_DEVERR_BAD_PATH, b);
        return;
    }
    const int64_t row_stride = (int64_t)hkv * ROW_BYTES;  // bytes per cache row
    const int64_t base = (ks + P) * row_stride + (int64_t)g * ROW_BYTES;
    gather_path<ROW_BYTES, kCompactThreads>(kc, vc, base, row_stride, sidx, L, max_depth, stage);
    if (g == 0 && tid == 0) new_len[b] = P + L;
}

// tree_accept_commit: the walk and the gather in one launch.  One workgroup
// per (request, KV head); its first wavefront walks the request's tree (every
// head's workgroup walks it, which costs less than a second launch), shares
// the path through LDS, and then all threads gather the head's rows.  The
// head-0 workgroup writes the walk's outputs and the new length.
template <int ROW_BYTES>
__global__ void __launch_bounds__(kCompactThreads) accept_commit_kernel(
    const int32_t *__restrict__ parent, const int32_t *__restrict__ draft,
    const int32_t *__restrict__ target, const int32_t *__restrict__ root_target,
    const int32_t *__restrict__ cu_nodes, const int32_t *__restrict__ kv_start,
    const int32_t *__restrict__ prefix_len, int total_nodes, int max_depth, int64_t kv_rows, int hkv,
    uint8_t *__restrict__ kc, uint8_t *__restrict__ vc, int32_t *__restrict__ accept_len,
    int32_t *__restrict__ accept_idx, int32_t *__restrict__ next_token,
    int32_t *__restrict__ new_len, int32_t *__restrict__ err) {
    extern __shared__ uint4 stage[];                                       // [2][max_depth][V16]
    __shared__ int32_t stg[TV_MAX_NODES];
    __shared__ int32_t sidx[TV_MAX_DEPTH];
    __shared__ int32_t s_len, s_next;
    const int b = blockIdx.x;
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    const bool walker = tid < 64;  // wave 0
    int lo;
    const int n = request_nodes(cu_nodes, b, total_nodes, total_nodes, &lo);
    const int root_want = root_target[b];
    const int P = prefix_len[b];
    const int64_t ks = kv_start[b];
    if ((n < 0) | (P < 0) | (ks < 0) | (ks + P + n > kv_rows)) {
        if (g == 0 && tid == 0) report(err, TV_DEVERR_BAD_REQUEST, b);
        return;
    }
    const int32_t *par = parent + lo;
    const int32_t *dr = draft + lo;
    const int32_t *tg = target + lo;
    const bool held = n <= TV_MAX_NODES;  // workgroup-uniform
    int pk[kWalkPerLane];
    int dk[kWalkPerLane];
    if (walker && held) walk_load(par, dr, tg, n, pk, dk, stg);
    __syncthreads();
    if (walker) {
        if (held) {
            int next;
            const int len = walk_registers(pk, dk, stg, n, root_want, max_depth, sidx, &next);
            if (tid == 0) {
                s_len = len;
                s_next = next;
            }
        } else {
            walk_global(par, dr, tg, n, root_want, max_depth, sidx, &s_len, &s_next);
        }
    }
    __syncthreads();
    const int L = s_len;
    if (g == 0) {
        for (int j = tid; j < max_depth; j += kCompactThreads) accept_idx[(int64_t)b * max_depth + j] = sidx[j];
        if (tid == 0) {
            accept_len[b] = L;
            next_token[b] = s_next;
            new_len[b] = P + L;
        }
    }
    const int64_t row_stride = (int64_t)hkv * ROW_BYTES;  // bytes per cache row
    const int64_t base = (ks + P) * row_stride + (int64_t)g * ROW_BYTES;
    gather_path<ROW_BYTES, kCompactThreads>(kc, vc, base, row_stride, sidx, L, max_depth, stage);
}

}  // namespace

hipError_t launch_kv_compact(void *k, void *v, const int32_t *cu_nodes, const int32_t *kv_start,
                             const int32_t *prefix_len, const int32_t *accept_len,
                             const int32_t *accept_idx, int batch, int total_nodes, int max_depth,
                             int64_t kv_rows, int hkv, int head_dim, tv_dtype dtype, int32_t *new_len,
                             int32_t *err, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    if (max_depth > TV_MAX_DEPTH) return hipErrorInvalidValue;
    const int row_bytes = head_dim * (dtype == TV_F32 ? 4 : 2);
    const size_t shmem = 2 * (size_t)max_depth * row_bytes;
    dim3 grid(batch, hkv);
#define TV_COMPACT(RB)                                                                           \
    hipLaunchKernelGGL(kv_compact_kernel<RB>, grid, dim3(kCompactThreads), shmem, stream,         \
                       (uint8_t *)k, (uint8_t *)v, cu_nodes, kv_start, prefix_len, accept_len,      \
                       accept_idx, total_nodes, max_depth, kv_rows, hkv, new_len, err)
    switch (row_bytes) {
        case 128: TV_COMPACT(128); break;
        case 256: TV_COMPACT(256); break;
        case 512: TV_COMPACT(512); break;
        default: return hipErrorInvalidValue;
    }
#undef TV_COMPACT
    return hipGetLastError();
}

hipError_t launch_accept_commit(const int32_t *parent, const int32_t *draft, const int32_t *target,
                                const int32_t *root_target, const int32_t *cu_nodes,
                                const int32_t *kv_start, const int32_t *prefix_len, int batch,
                                int total_nodes, int max_depth, int64_t kv_rows, int hkv, int head_dim,
                                tv_dtype dtype, void *k, void *v, int32_t *accept_len,
                                int32_t *accept_idx, int32_t *next_token, int32_t *new_len, int32_t *err,
                                hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    if (max_depth > TV_MAX_DEPTH) return hipErrorInvalidValue;
    const int row_bytes = head_dim * (dtype == TV_F32 ? 4 : 2);
    const size_t shmem = 2 * (size_t)max_depth * row_bytes;
    dim3 grid(batch, hkv);
#define TV_COMMIT(RB)                                                                            \
    hipLaunchKernelGGL(accept_commit_kernel<RB>, grid, dim3(kCompactThreads), shmem, stream,      \
                       parent, draft, target, root_target, cu_nodes, kv_start, prefix_len,          \
                       total_nodes, max_depth, kv_rows, hkv, (uint8_t *)k, (uint8_t *)v, accept_len, \
                       accept_idx, next_token, new_len, err)
    switch (row_bytes) {
        case 128: TV_COMMIT(128); break;
        case 256: TV_COMMIT(256); break;
        case 512: TV_COMMIT(512); break;
        default: return hipErrorInvalidValue;
    }
#undef TV_COMMIT
    return hipGetLastError();
}

}  // namespace tv
