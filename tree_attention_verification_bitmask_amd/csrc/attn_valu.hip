// tree_attn_verify, fp32 path: vector (VALU) arithmetic over tiles of rows.
//
// [TSD] = "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
// Tree Attention Accelerate LLM Serving" (llms.blog), section "The Tree
// Attention Mechanism": each node attends to the whole prefix and to the tree
// nodes on its own root-to-node branch (parts 1 and 2).
//
// This path serves fp32 inputs (bf16 calls take the matrix-core kernel).  A
// workgroup owns a tile of R nodes x GQ query heads that share one KV head,
// so each K and V row it reads serves R * GQ rows.  The key axis is dealt over
// the workgroup's W wavefronts in chunks of 64 keys (chunk c to wave c mod
// W), one key per lane: the lane computes its key's logit against each row's
// q (held in LDS and read as a broadcast), the wave reduces max and sum per
// row (online softmax), and then every lane accumulates its own output
// channels over the chunk's visible keys, reading each V row coalesced once
// and each probability from its key's lane.  At the end the waves' (max, sum,
// output) are merged through LDS.  Tree keys j > i are never ancestors of node
// i (parents precede children), so node i's keys stop at P + i + 1.  All
// arithmetic is fp32; exp is expf.
//
// Optional inputs: with a token table the cache row of key position p is
// req_to_token[b][p] (each lane looks up its own key; the V loop takes key
// u's row from lane u); with RoPE on, q is rotated as it is staged in LDS,
// from the per-node (cos, sin) pairs that the RoPE pre-pass stored.
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {
namespace {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
    static __device__ __forceinline__ float ld(const float *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void st(float *p, int64_t i, float x) { p[i] = x; }
};
// 8 consecutive elements of a row starting at element e (32 bytes) -> fp32.
template <typename T>
__device__ __forceinline__ void load8(const T *row, int e, float out[8]);
template <>
__device__ __forceinline__ void load8<float>(const float *row, int e, float out[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(row + e);
    const float4 c = *reinterpret_cast<const float4 *>(row + e + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = c.x; out[5] = c.y; out[6] = c.z; out[7] = c.w;
}
// One workgroup per (R consecutive nodes, GQ consecutive query heads of one
// KV head, request).  Lane `lane` of a wave holds key c0 + lane and its R * GQ
// logits (row r = node i0 + r / GQ, query head h0 + r % GQ); the V loop reads
// each key's row once, skips keys that no row of the tile sees, and adds the
// row to every row's output with the probability read from the key's lane.
template <typename T, int D, int W, int GQ, int R>
__global__ void __launch_bounds__(64 * W) attn_valu_tile_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const int32_t *__restrict__ cu_nodes, const int32_t *__restrict__ kv_start,
    const int32_t *__restrict__ prefix_len, const uint64_t *__restrict__ anc, int total_nodes,
    int max_nodes, int max_prefix, int64_t kv_rows, int hq, int hkv, float scale, T *__restrict__ out,
    int32_t *__restrict__ err, const int32_t *__restrict__ table, int64_t table_stride,
    const float2 *__restrict__ rope_cs) {
    constexpr int CPL = D / 64;  // output channels per lane
    constexpr int ROWS = GQ * R;
    __shared__ float qs[ROWS][D];
    __shared__ float wm[W][ROWS], wl[W][ROWS];
    __shared__ float wacc[W][ROWS][D];
    const int i0 = blockIdx.x * R;  // first request-local node of the tile
    const int h0 = blockIdx.y * GQ; // first query head of the tile
    const int g = h0 / (hq / hkv);  // their KV head (GQ divides the group)
    const int b = blockIdx.z;       // request
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int lo;
    const int n = request_nodes(cu_nodes, b, total_nodes, max_nodes, &lo);
    const int P = prefix_len[b];
    const int64_t ks = table ? 0 : kv_start[b];
    const bool rows_bad = table ? ((int64_t)P + n > table_stride) : (ks < 0 || ks + P + n > kv_rows);
    if (n < 0 || P < 0 || P > max_prefix || rows_bad) {
        if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) report(err, TV_DEVERR_BAD_REQUEST, b);
        return;
    }
    if (i0 >= n) return;
    const int nr = min(R, n - i0);  // nodes of the tile that exist
    const int words = (max_nodes + 63) / 64;
    const int64_t t0 = (int64_t)lo + i0;

    for (int e = tid; e < ROWS * (D / 2); e += 64 * W) {
        const int r = e / (D / 2), c = e % (D / 2);
        const int ri = min(r / GQ, nr - 1);  // rows past the tree repeat a valid node (never stored)
        const int64_t t = t0 + ri;
        const int64_t qrow = (t * hq + h0 + r % GQ) * D;
        const float x1 = Elem<T>::ld(q, qrow + c);
        const float x2 = Elem<T>::ld(q, qrow + c + D / 2);
        if (rope_cs) {
            // channel c paired with c + D/2, rotated in fp32 by the node's angle
            const float2 cs = rope_cs[t * (D / 2) + c];
            qs[r][c] = x1 * cs.x - x2 * cs.y;
            qs[r][c + D / 2] = x2 * cs.x + x1 * cs.y;
        } else {
            qs[r][c] = x1;
            qs[r][c + D / 2] = x2;
        }
    }
    __syncthreads();

    const int64_t kv_stride = (int64_t)hkv * D;  // elements per cache row
    const T *kbase = k + (int64_t)g * D;
    const T *vbase = v + (int64_t)g * D;
    const int32_t *trow = table ? table + (int64_t)b * table_stride : nullptr;
    const int nkeys = P + i0 + nr;  // keys of the tile's last node

    float m[ROWS], l[ROWS], acc[ROWS][CPL];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[r][c] = 0.f;
    }

    for (int c0 = 64 * wv; c0 < nkeys; c0 += 64 * W) {
        const int key = c0 + lane;
        // visibility of this lane's key to each node of the tile: the whole
        // prefix, then the node's ancestors (itself included) among the tree
        bool okn[R];
#pragma unroll
        for (int ri = 0; ri < R; ++ri) {
            bool ok = ri < nr && key < P + i0 + ri + 1;
            if (ok && key >= P) {
                const int j = key - P;
                ok = (anc[(t0 + ri) * words + (j >> 6)] >> (j & 63)) & 1ull;
            }
            okn[ri] = ok;
        }
        bool any = false;
#pragma unroll
        for (int ri = 0; ri < R; ++ri) any = any || okn[ri];
        // cache row of this lane's key (key u's row is read from lane u below)
        int64_t krow = ks + key;
        if (trow && key < nkeys) {
            krow = trow[key];
            if (krow < 0 || krow >= kv_rows) {
                report(err, TV_DEVERR_BAD_SLOT, b);
                krow = 0;
            }
        }
        float s[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) s[r] = 0.f;
        if (any) {
            const T *kr = kbase + krow * kv_stride;
#pragma unroll 2
            for (int e = 0; e < D; e += 8) {
                float kk[8];
                load8<T>(kr, e, kk);
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
#pragma unroll
                    for (int u = 0; u < 8; ++u) s[r] = fmaf(qs[r][e + u], kk[u], s[r]);
            }
        }
        float p[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const bool ok = okn[r / GQ];
            const float sh = ok ? s[r] * scale : -INFINITY;
            const float mn = fmaxf(m[r], wave_max(sh));
            // A chunk can be fully masked for a row (P == 0 and none of its
            // nodes is an ancestor); while no finite logit has been seen, use
            // 0 as the reference so that nothing evaluates exp(-inf - -inf).
            const float mref = (mn == -INFINITY) ? 0.f : mn;
            const float alpha = expf(m[r] - mref);
            p[r] = ok ? expf(sh - mref) : 0.f;
            l[r] = l[r] * alpha + wave_sum(p[r]);
            m[r] = mn;
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[r][c] *= alpha;
        }
        const uint64_t seen = __ballot(any);  // keys some row of the tile sees
        const int klo = (int)(uint32_t)krow, khi = (int)(uint32_t)((uint64_t)krow >> 32);
        for (uint64_t bits = seen; bits; bits &= bits - 1) {
            const int u = __builtin_ctzll(bits);
            const uint64_t ru = (uint32_t)__builtin_amdgcn_readlane(klo, u) |
                                ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(khi, u) << 32);
            const T *vr = vbase + (int64_t)ru * kv_stride;
            float vv[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) vv[c] = Elem<T>::ld(vr, lane + 64 * c);
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const float pu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[r]), u));
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[r][c] = fmaf(pu, vv[c], acc[r][c]);
            }
        }
    }
    // merge the waves, per row: M = max m_w, out = sum_w e^(m_w - M) acc_w /
    // sum_w e^(m_w - M) l_w (a wave that saw no visible key has l = 0 and adds
    // nothing)
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            wm[wv][r] = m[r];
            wl[wv][r] = l[r];
        }
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int c = 0; c < CPL; ++c) wacc[wv][r][lane + 64 * c] = acc[r][c];
    __syncthreads();
    for (int e = tid; e < nr * GQ * D; e += 64 * W) {
        const int r = e / D, ch = e % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, wm[w][r]);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            if (wl[w][r] > 0.f) {
                const float a = expf(wm[w][r] - M);
                L = fmaf(a, wl[w][r], L);
                o = fmaf(a, wacc[w][r][ch], o);
            }
        }
        Elem<T>::st(out, ((t0 + r / GQ) * hq + h0 + r % GQ) * D + ch, o / L);
    }
}

template <typename T, int D, int W, int GQ, int R>
hipError_t launch_tile(const AttnArgs &a, hipStream_t stream) {
    dim3 grid((a.max_nodes + R - 1) / R, a.hq / GQ, a.batch);
    hipLaunchKernelGGL((attn_valu_tile_kernel<T, D, W, GQ, R>), grid, dim3(64 * W), 0, stream, (const T *)a.q,
                       (const T *)a.k, (const T *)a.v, a.cu_nodes, a.kv_start, a.prefix_len, a.anc,
                       a.total_nodes, a.max_nodes, a.max_prefix, a.kv_rows, a.hq, a.hkv, a.scale,
                       (T *)a.out, a.err, a.table, a.table_stride, a.rope_cs);
    return hipGetLastError();
}
// Nodes per tile: the most (4, 2 or 1) that keep R * GQ <= 16 rows (register
// budget) and still leave kTileMinWgs workgroups for the 256 CUs.  Eight waves
// per workgroup; sixteen for an untiled grid over a long key axis, where the
// workgroups are few and each needs more keys in flight (not for GQ 8, whose
// per-wave partials would fill the LDS).  Measured, fp32, 32 query / 8 KV
// heads, d 128, us per call (R 1 / R 2 / R 4): 64 nodes over 1024 keys 79 /
// 78 / 105; 128 nodes over 4096 keys 523 / - / 341; 4 requests of 32 nodes
// over 2048 keys 276 / - / 195.
constexpr long kTileMinWgs = 256;
template <typename T, int D, int GQ>
hipError_t launch_group(const AttnArgs &a, hipStream_t stream) {
    const long per_node = (long)(a.hq / GQ) * a.batch;  // workgroups per node of the grid
    auto wgs = [&](int r) { return (long)((a.max_nodes + r - 1) / r) * per_node; };
    if constexpr (4 * GQ <= 16) {
        if (wgs(4) >= kTileMinWgs) return launch_tile<T, D, 8, GQ, 4>(a, stream);
    }
    if constexpr (2 * GQ <= 16) {
        if (wgs(2) >= kTileMinWgs) return launch_tile<T, D, 8, GQ, 2>(a, stream);
    }
    if constexpr (GQ < 8) {
        if ((int64_t)a.max_prefix + a.max_nodes >= 4096) return launch_tile<T, D, 16, GQ, 1>(a, stream);
    }
    return launch_tile<T, D, 8, GQ, 1>(a, stream);
}
// GQ: the largest divisor of the GQA group size hq / hkv up to 8.
template <typename T, int D>
hipError_t launch_typed(const AttnArgs &a, hipStream_t stream) {
    const int G = a.hq / a.hkv;
    if (G % 8 == 0) return launch_group<T, D, 8>(a, stream);
    if (G % 7 == 0) return launch_group<T, D, 7>(a, stream);
    if (G % 6 == 0) return launch_group<T, D, 6>(a, stream);
    if (G % 5 == 0) return launch_group<T, D, 5>(a, stream);
    if (G % 4 == 0) return launch_group<T, D, 4>(a, stream);
    if (G % 3 == 0) return launch_group<T, D, 3>(a, stream);
    if (G % 2 == 0) return launch_group<T, D, 2>(a, stream);
    return launch_group<T, D, 1>(a, stream);
}

}  // namespace

hipError_t launch_attn_valu(const AttnArgs &a, hipStream_t stream) {
    if (a.batch == 0 || a.max_nodes == 0) return hipSuccess;
    // bf16 calls with work always take the matrix-core kernel
    if (a.dtype != TV_F32) return hipErrorInvalidValue;
    return a.head_dim == 64 ? launch_typed<float, 64>(a, stream) : launch_typed<float, 128>(a, stream);
}

}  // namespace tv
