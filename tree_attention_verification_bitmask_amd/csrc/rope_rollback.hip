// tree_rope_apply and kv_rollback_token_table.
//
// [TSD] = "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
// Tree Attention Accelerate LLM Serving" (llms.blog): "The Tree Attention
// Mechanism", part 3 "Tree Positional IDs" (the position a node's RoPE sees is
// PosID(root) + depth) and "KV Cache Rollback" (unaccepted nodes are dropped
// by page-table updates in paged caches).
//
// tree_rope_apply: one thread per (row, channel pair) over the queries and
// the tree's K rows of every request, in one launch.  The angle
// pos * base^(-2i/d), its sine and cosine and the rotation are taken in
// double and the result is rounded to the element type: streaming work, one
// read and one write of every rotated element.  A K row finds its request by
// a binary search over cu_nodes.
//
// rope_prep_kernel (RoPE inside tree_attn_verify_ex): one thread per (node,
// channel pair) takes the same angle, sine and cosine in double, stores the
// pair as fp32 (the attention kernel rotates q with it as q is loaded) and
// rotates the node's K row of every KV head in place exactly as rope_kernel
// does, so the cache ends up bit for bit as after tree_rope_apply.  The K row
// is found from kv_start or through the token table.
//
// kv_rollback_token_table: one wavefront per request.  Lane j < L writes
// position P + j of the request's token table; the unaccepted nodes' slots are
// compacted in node order with one ballot per 64 nodes.
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {
namespace {

constexpr int kRopeThreads = 256;

template <typename T>
__device__ __forceinline__ double load_el(const T *p);
template <>
__device__ __forceinline__ double load_el<float>(const float *p) { return (double)*p; }
template <>
__device__ __forceinline__ double load_el<uint16_t>(const uint16_t *p) {
    return (double)__uint_as_float((uint32_t)*p << 16);
}
template <typename T>
__device__ __forceinline__ void store_el(T *p, double v);
template <>
__device__ __forceinline__ void store_el<float>(float *p, double v) { *p = (float)v; }
template <>
__device__ __forceinline__ void store_el<uint16_t>(uint16_t *p, double v) {
    // to float, then to bf16 (round to nearest even): within one bf16 ulp of
    // the exact result
    const uint32_t u = __float_as_uint((float)v);
    *p = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Work item w covers (row, pair): rows 0 .. T*hq-1 are query rows (node t =
// row / hq), the next T*hkv rows are tree K rows (node t = row / hkv).
template <typename T>
__global__ void __launch_bounds__(kRopeThreads) rope_kernel(
    T *__restrict__ q, T *__restrict__ k, const int32_t *__restrict__ pos, const int32_t *__restrict__ cu_nodes,
    const int32_t *__restrict__ kv_start, const int32_t *__restrict__ prefix_len, int batch, int total_nodes,
    int64_t kv_rows, int hq, int hkv, int d, double log2_base, int32_t *__restrict__ err) {
    const int h = d / 2;
    const int64_t w = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
    const int64_t qrows = (int64_t)total_nodes * hq;
    const int64_t nrows = qrows + (int64_t)total_nodes * hkv;
    if (w >= nrows * h) return;
    const int64_t row = w / h;
    const int i = (int)(w - row * h);
    T *base;
    int t;
    if (row < qrows) {
        t = (int)(row / hq);
        base = q + row * d;
    } else {
        const int64_t kr = row - qrows;
        t = (int)(kr / hkv);
        const int g = (int)(kr - (int64_t)t * hkv);
        const int b = request_of(cu_nodes, batch, t);
        if (b < 0) {
            report(err, TV_DEVERR_BAD_REQUEST, 0);
            return;
        }
        const int64_t crow = (int64_t)kv_start[b] + prefix_len[b] + (t - cu_nodes[b]);
        if (crow < 0 || crow >= kv_rows || kv_start[b] < 0 || prefix_len[b] < 0) {
            report(err, TV_DEVERR_BAD_REQUEST, b);
            return;
        }
        base = k + (crow * hkv + g) * d;
    }
    const double inv = exp2(-2.0 * i / d * log2_base);
    const double ang = (double)pos[t] * inv;
    double s, c;
    sincos(ang, &s, &c);
    const double a = load_el<T>(base + i), bb = load_el<T>(base + i + h);
    store_el<T>(base + i, a * c - bb * s);
    store_el<T>(base + i + h, bb * c + a * s);
}

template <typename T>
__global__ void __launch_bounds__(kRopeThreads) rope_prep_kernel(
    T *__restrict__ k, const int32_t *__restrict__ pos, const int32_t *__restrict__ cu_nodes,
    const int32_t *__restrict__ kv_start, const int32_t *__restrict__ prefix_len, const int32_t *__restrict__ table,
    int64_t table_stride, int batch, int total_nodes, int64_t kv_rows, int hkv, int d, double log2_base,
    float2 *__restrict__ cs, int32_t *__restrict__ err) {
    const int h = d / 2;
    const int64_t w = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
    if (w >= (int64_t)total_nodes * h) return;
    const int t = (int)(w / h);
    const int i = (int)(w - (int64_t)t * h);
    const double inv = exp2(-2.0 * i / d * log2_base);
    const double ang = (double)pos[t] * inv;
    double s, c;
    sincos(ang, &s, &c);
    cs[w] = make_float2((float)c, (float)s);
    const int b = request_of(cu_nodes, batch, t);
    if (b < 0) {
        report(err, TV_DEVERR_BAD_REQUEST, 0);
        return;
    }
    const int j = t - cu_nodes[b];
    const int P = prefix_len[b];
    int64_t crow;
    if (table) {
        if (P < 0 || (int64_t)P + (cu_nodes[b + 1] - cu_nodes[b]) > table_stride) {
            report(err, TV_DEVERR_BAD_REQUEST, b);
            return;
        }
        crow = table[(int64_t)b * table_stride + P + j];
        if (crow < 0 || crow >= kv_rows) {
            report(err, TV_DEVERR_BAD_SLOT, b);
            return;
        }
    } else {
        crow = (int64_t)kv_start[b] + P + j;
        if (crow < 0 || crow >= kv_rows || kv_start[b] < 0 || P < 0) {
            report(err, TV_DEVERR_BAD_REQUEST, b);
            return;
        }
    }
    for (int g = 0; g < hkv; ++g) {
        T *base = k + (crow * hkv + g) * d;
        const double a = load_el<T>(base + i), bb = load_el<T>(base + i + h);
        store_el<T>(base + i, a * c - bb * s);
        store_el<T>(base + i + h, bb * c + a * s);
    }
}

__global__ void __launch_bounds__(64) rollback_kernel(
    int32_t *__restrict__ table, int64_t stride, const int32_t *__restrict__ tree_slots,
    const int32_t *__restrict__ cu_nodes, const int32_t *__restrict__ prefix_len,
    const int32_t *__restrict__ accept_len, const int32_t *__restrict__ accept_idx, int total_nodes,
    int max_depth, int32_t *__restrict__ new_len, int32_t *__restrict__ freed, int32_t *__restrict__ n_freed,
    int32_t *__restrict__ err) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    int lo;
    const int n = request_nodes(cu_nodes, b, total_nodes, total_nodes, &lo);
    const int P = prefix_len[b];
    const int L = accept_len[b];
    // the path row is read with the sizes (in bounds whatever they are), and
    // the checks use no short-circuit: one memory round trip, not four
    const int32_t *idx = accept_idx + (int64_t)b * max_depth;
    const int my_raw = lane < max_depth ? idx[lane] : -1;  // TV_MAX_DEPTH == 64 == lanes
    if ((n < 0) | (P < 0) | (L < 0) | (L > max_depth) | (L > n) | ((int64_t)P + L > stride)) {
        if (lane == 0) report(err, TV_DEVERR_BAD_REQUEST, b);
        return;
    }
    const int my = lane < L ? my_raw : -1;
    if (__ballot(lane < L && (my < 0 || my >= n)) != 0) {
        if (lane == 0) report(err, TV_DEVERR_BAD_PATH, b);
        return;
    }
    if (lane < L) table[(int64_t)b * stride + P + lane] = tree_slots[lo + my];
    // unaccepted nodes, in node order
    int out = 0;
    for (int base = 0; base < n; base += 64) {
        const int i = base + lane;
        bool acc = false;
        for (int j = 0; j < L; ++j) acc |= __shfl(my, j, 64) == i;
        const bool keep = i < n && !acc;
        const unsigned long long bal = __ballot(keep);
        if (keep) freed[lo + out + __popcll(bal & ((1ull << lane) - 1ull))] = tree_slots[lo + i];
        out += __popcll(bal);
    }
    for (int i = out + lane; i < n; i += 64) freed[lo + i] = -1;
    if (lane == 0) {
        new_len[b] = P + L;
        n_freed[b] = out;
    }
}

}  // namespace

hipError_t launch_tree_rope(void *q, void *k, const int32_t *pos, const int32_t *cu_nodes, const int32_t *kv_start,
                            const int32_t *prefix_len, int batch, int total_nodes, int64_t kv_rows, int hq, int hkv,
                            int head_dim, float base, tv_dtype dtype, int32_t *err, hipStream_t stream) {
    if (batch == 0 || total_nodes == 0) return hipSuccess;
    const int64_t items = (int64_t)total_nodes * (hq + hkv) * (head_dim / 2);
    const int64_t blocks = (items + kRopeThreads - 1) / kRopeThreads;
    const double lb = log2((double)base);
    if (dtype == TV_BF16)
        hipLaunchKernelGGL(rope_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kRopeThreads), 0, stream,
                           (uint16_t *)q, (uint16_t *)k, pos, cu_nodes, kv_start, prefix_len, batch, total_nodes,
                           kv_rows, hq, hkv, head_dim, lb, err);
    else
        hipLaunchKernelGGL(rope_kernel<float>, dim3((unsigned)blocks), dim3(kRopeThreads), 0, stream, (float *)q,
                           (float *)k, pos, cu_nodes, kv_start, prefix_len, batch, total_nodes, kv_rows, hq, hkv,
                           head_dim, lb, err);
    return hipGetLastError();
}

hipError_t launch_rope_prep(void *k, const int32_t *pos, const int32_t *cu_nodes, const int32_t *kv_start,
                            const int32_t *prefix_len, const int32_t *table, int64_t table_stride, int batch,
                            int total_nodes, int64_t kv_rows, int hkv, int head_dim, float base, tv_dtype dtype,
                            float2 *cs, int32_t *err, hipStream_t stream) {
    if (batch == 0 || total_nodes == 0) return hipSuccess;
    const int64_t items = (int64_t)total_nodes * (head_dim / 2);
    const int64_t blocks = (items + kRopeThreads - 1) / kRopeThreads;
    const double lb = log2((double)base);
    if (dtype == TV_BF16)
        hipLaunchKernelGGL(rope_prep_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kRopeThreads), 0, stream,
                           (uint16_t *)k, pos, cu_nodes, kv_start, prefix_len, table, table_stride, batch,
                           total_nodes, kv_rows, hkv, head_dim, lb, cs, err);
    else
        hipLaunchKernelGGL(rope_prep_kernel<float>, dim3((unsigned)blocks), dim3(kRopeThreads), 0, stream,
                           (float *)k, pos, cu_nodes, kv_start, prefix_len, table, table_stride, batch,
                           total_nodes, kv_rows, hkv, head_dim, lb, cs, err);
    return hipGetLastError();
}

hipError_t launch_rollback_table(int32_t *table, int64_t stride, const int32_t *tree_slots, const int32_t *cu_nodes,
                                 const int32_t *prefix_len, const int32_t *accept_len, const int32_t *accept_idx,
                                 int batch, int total_nodes, int max_depth, int32_t *new_len, int32_t *freed,
                                 int32_t *n_freed, int32_t *err, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    hipLaunchKernelGGL(rollback_kernel, dim3(batch), dim3(64), 0, stream, table, stride, tree_slots, cu_nodes,
                       prefix_len, accept_len, accept_idx, total_nodes, max_depth, new_len, freed, n_freed, err);
    return hipGetLastError();
}

}  // namespace tv
