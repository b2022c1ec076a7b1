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
// A grid of few tiles (a few nodes, a long prefix) cuts the key axis into
// slices, one workgroup each: a slice's workgroup writes its rows' (max, sum,
// unnormalised output) to the workspace, and attn_valu_merge_kernel combines
// the slices of each row, as the waves of a workgroup are combined.
//
// Optional inputs: with a token table the cache row of key position p is
// req_to_token[b][p] (each lane looks up its own key; the V loop takes key
// u's row from lane u); with RoPE on, q is rotated as it is staged in LDS,
// from the per-node (cos, sin) pairs that the RoPE pre-pass stored.
#include <algorithm>

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
    const float2 *__restrict__ rope_cs, int splits, int keys_per_split, float2 *__restrict__ part_ml,
    float *__restrict__ part_o) {
    constexpr int CPL = D / 64;  // output channels per lane
    constexpr int ROWS = GQ * R;
    __shared__ float qs[ROWS][D];
    __shared__ float wm[W][ROWS], wl[W][ROWS];
    __shared__ float wacc[W][ROWS][D];
    const int split = blockIdx.x % splits;  // key-axis slice (0 when unsliced)
    const int i0 = blockIdx.x / splits * R;  // first request-local node of the tile
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
    // the slice's keys, up to those of the tile's last node
    const int kbeg = split * keys_per_split;
    const int kend = splits > 1 ? min(P + i0 + nr, kbeg + keys_per_split) : P + i0 + nr;

    float m[ROWS], l[ROWS], acc[ROWS][CPL];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[r][c] = 0.f;
    }

    for (int c0 = kbeg + 64 * wv; c0 < kend; c0 += 64 * W) {
        const int key = c0 + lane;
        // visibility of this lane's key to each node of the tile: the whole
        // prefix, then the node's ancestors (itself included) among the tree
        bool okn[R];
#pragma unroll
        for (int ri = 0; ri < R; ++ri) {
            bool ok = ri < nr && key < kend && key < P + i0 + ri + 1;
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
        if (trow && key < kend) {
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
        const int64_t row = (t0 + r / GQ) * hq + h0 + r % GQ;
        if (splits == 1) {
            Elem<T>::st(out, row * D + ch, o / L);
        } else {
            // a slice with no visible key writes (-inf, 0, 0)
            part_o[(row * splits + split) * D + ch] = o;
            if (ch == 0) part_ml[row * splits + split] = make_float2(M, L);
        }
    }
}

// Combines the key-axis slices of each (node, query head) row: one workgroup
// of D threads per row, one output channel per thread.  M = max of the
// slices' maxima, out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s (every
// row sees at least its own node, so the sum is positive).  Requests that the
// tile kernel rejected (and reported) are skipped here too.
template <typename T, int D>
__global__ void __launch_bounds__(D) attn_valu_merge_kernel(
    const int32_t *__restrict__ cu_nodes, const int32_t *__restrict__ kv_start,
    const int32_t *__restrict__ prefix_len, int total_nodes, int max_nodes, int max_prefix, int64_t kv_rows,
    int hq, const int32_t *__restrict__ table, int64_t table_stride, int splits,
    const float2 *__restrict__ part_ml, const float *__restrict__ part_o, T *__restrict__ out) {
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, ch = threadIdx.x;
    int lo;
    const int n = request_nodes(cu_nodes, b, total_nodes, max_nodes, &lo);
    const int P = prefix_len[b];
    const int64_t ks = table ? 0 : kv_start[b];
    const bool rows_bad = table ? ((int64_t)P + n > table_stride) : (ks < 0 || ks + P + n > kv_rows);
    if (n < 0 || P < 0 || P > max_prefix || rows_bad || i >= n) return;
    const int64_t row = ((int64_t)lo + i) * hq + h;
    const float2 *ml = part_ml + row * splits;
    const float *po = part_o + row * splits * D + ch;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[s].x);
    float L = 0.f, o = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float2 x = ml[s];
        if (x.y > 0.f) {
            const float a = expf(x.x - M);
            L = fmaf(a, x.y, L);
            o = fmaf(a, po[(int64_t)s * D], o);
        }
    }
    Elem<T>::st(out, row * D + ch, o / L);
}

// Key-axis slices of a launch: count, keys per slice, and the workspace
// arrays of the slices' (max, sum) and outputs (null when unsliced).
struct Slices {
    int count = 1, keys = 0;
    float2 *ml = nullptr;
    float *o = nullptr;
};

template <typename T, int D, int W, int GQ, int R>
hipError_t launch_tile(const AttnArgs &a, const Slices &sl, hipStream_t stream) {
    dim3 grid((a.max_nodes + R - 1) / R * sl.count, a.hq / GQ, a.batch);
    hipLaunchKernelGGL((attn_valu_tile_kernel<T, D, W, GQ, R>), grid, dim3(64 * W), 0, stream, (const T *)a.q,
                       (const T *)a.k, (const T *)a.v, a.cu_nodes, a.kv_start, a.prefix_len, a.anc,
                       a.total_nodes, a.max_nodes, a.max_prefix, a.kv_rows, a.hq, a.hkv, a.scale,
                       (T *)a.out, a.err, a.table, a.table_stride, a.rope_cs, sl.count, sl.keys, sl.ml, sl.o);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || sl.count == 1) return e;
    hipLaunchKernelGGL((attn_valu_merge_kernel<T, D>), dim3(a.max_nodes, a.hq, a.batch), dim3(D), 0, stream,
                       a.cu_nodes, a.kv_start, a.prefix_len, a.total_nodes, a.max_nodes, a.max_prefix,
                       a.kv_rows, a.hq, a.table, a.table_stride, sl.count, sl.ml, sl.o, (T *)a.out);
    return hipGetLastError();
}
// Nodes per tile: the most (4, 2 or 1) that keep R * GQ <= 16 rows (register
// budget) and still leave kTileMinWgs workgroups for the 256 CUs.  Eight waves
// per workgroup; sixteen for an untiled, unsliced grid over a long key axis,
// where each workgroup needs more keys in flight (not for GQ 8, whose
// per-wave partials would fill the LDS).  Measured, fp32, 32 query / 8 KV
// heads, d 128, us per call (R 1 / R 2 / R 4): 64 nodes over 1024 keys 79 /
// 78 / 105; 128 nodes over 4096 keys 523 / - / 341; 4 requests of 32 nodes
// over 2048 keys 276 / - / 195.
constexpr long kTileMinWgs = 256;
// A grid of at least kManyWgs 4-node tiles (slices counted) runs them as
// 4-wave workgroups: at about 150 VGPRs a CU then holds three workgroups (12
// waves) instead of one 8-wave workgroup, and hides more of the K/V reads'
// latency.  A grid of at most kTileMinWgs such tiles over a key axis of at
// least 2 * kMinOccSliceKeys is cut into slices to get there.  Measured, fp32,
// us per call: c5 (2016 tiles) 3324 with 8 waves, 2269 with 4; c3 (256 tiles,
// 4224 keys) 404 unsliced, 336 in 3 slices; c4 (512 tiles) 1573 unsliced,
// 1608 in 2 slices, so it stays unsliced with 8 waves.
constexpr long kManyWgs = 768;
constexpr long kMinOccSliceKeys = 1024;
// A grid of fewer than kTileMinWgs one-node tiles whose key axis holds at
// least two slices of kMinSliceKeys keys is cut into slices, as many as bring
// it to kSliceWgs workgroups; its tiles then take as many nodes as the rows
// allow, since the slices restore the parallelism and larger tiles read each
// K/V row fewer times.  Measured, fp32, 32 query / 8 KV heads, d 128, us per
// call (one-node tiles unsliced / sliced / largest tiles sliced): 1 node over
// 8192 keys 279 / 46 / 46; 7 nodes over 8192 keys 283 / 147 / 95.  Slicing
// to 512 or 1024 workgroups, or into slices of 128 keys, was slower for
// every such shape tried except 1 node over 32768 keys (106 against 118).
constexpr long kSliceWgs = 256;
constexpr long kMinSliceKeys = 256;

// GQ: the largest divisor of the GQA group size hq / hkv up to 8.
int group_tile(int G) {
    for (int x = 8; x > 1; --x)
        if (G % x == 0) return x;
    return 1;
}
bool sliced_grid(int max_nodes, int max_prefix, int hq, int gq, int batch) {
    return (long)max_nodes * (hq / gq) * batch < kTileMinWgs &&
           (long)max_prefix + max_nodes >= 2 * kMinSliceKeys;
}
int nodes_per_tile(int max_nodes, int max_prefix, int hq, int gq, int batch) {
    const long per_node = (long)(hq / gq) * batch;  // workgroups per node of the grid
    const bool sliced = sliced_grid(max_nodes, max_prefix, hq, gq, batch);
    for (int r = 4; r > 1; r /= 2) {
        if (r * gq > 16) continue;
        if (sliced ? r / 2 < max_nodes : (long)((max_nodes + r - 1) / r) * per_node >= kTileMinWgs) return r;
    }
    return 1;
}

template <typename T, int D, int GQ>
hipError_t launch_group(const AttnArgs &a, const Slices &sl, hipStream_t stream) {
    const int r = nodes_per_tile(a.max_nodes, a.max_prefix, a.hq, GQ, a.batch);
    if constexpr (4 * GQ <= 16) {
        if (r == 4) {
            if ((long)((a.max_nodes + 3) / 4) * (a.hq / GQ) * a.batch * sl.count >= kManyWgs)
                return launch_tile<T, D, 4, GQ, 4>(a, sl, stream);
            return launch_tile<T, D, 8, GQ, 4>(a, sl, stream);
        }
    }
    if constexpr (2 * GQ <= 16) {
        if (r == 2) return launch_tile<T, D, 8, GQ, 2>(a, sl, stream);
    }
    if constexpr (GQ < 8) {
        if (sl.count == 1 && (int64_t)a.max_prefix + a.max_nodes >= 4096)
            return launch_tile<T, D, 16, GQ, 1>(a, sl, stream);
    }
    return launch_tile<T, D, 8, GQ, 1>(a, sl, stream);
}
template <typename T, int D>
hipError_t launch_typed(const AttnArgs &a, const Slices &sl, hipStream_t stream) {
    switch (group_tile(a.hq / a.hkv)) {
        case 8: return launch_group<T, D, 8>(a, sl, stream);
        case 7: return launch_group<T, D, 7>(a, sl, stream);
        case 6: return launch_group<T, D, 6>(a, sl, stream);
        case 5: return launch_group<T, D, 5>(a, sl, stream);
        case 4: return launch_group<T, D, 4>(a, sl, stream);
        case 3: return launch_group<T, D, 3>(a, sl, stream);
        case 2: return launch_group<T, D, 2>(a, sl, stream);
        default: return launch_group<T, D, 1>(a, sl, stream);
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

void plan_attn_valu(int batch, int total_nodes, int max_nodes, int max_prefix, int hq, int hkv, int head_dim,
                    const tv_attn_plan_override *ov, MfmaPlan *plan) {
    plan->splits = 1;
    plan->keys_per_split = 0;
    plan->ws_bytes = 0;
    if (batch <= 0 || max_nodes <= 0 || total_nodes <= 0 || hkv <= 0 || hq < hkv) return;
    const int gq = group_tile(hq / hkv);
    const int r = nodes_per_tile(max_nodes, max_prefix, hq, gq, batch);
    const long span = (long)max_prefix + max_nodes;  // longest key axis
    const long wgs = (long)((max_nodes + r - 1) / r) * (hq / gq) * batch;
    long s = 1;
    if (ov && ov->splits > 0)
        s = std::min<long>(ov->splits, (span + 63) / 64);
    else if (sliced_grid(max_nodes, max_prefix, hq, gq, batch))
        s = std::min<long>((kSliceWgs + wgs - 1) / wgs, span / kMinSliceKeys);
    else if (r == 4 && wgs <= kTileMinWgs && span >= 2 * kMinOccSliceKeys)
        s = std::min<long>((kManyWgs + wgs - 1) / wgs, span / kMinOccSliceKeys);
    if (s <= 1) return;
    const long keys = ((span + s - 1) / s + 63) / 64 * 64;  // whole 64-key chunks
    s = (span + keys - 1) / keys;
    if (s <= 1) return;
    plan->splits = (int)s;
    plan->keys_per_split = (int)keys;
    const size_t rows = (size_t)total_nodes * hq * s;
    plan->ws_bytes = align256(rows * sizeof(float2)) + rows * head_dim * sizeof(float);
}

hipError_t launch_attn_valu(const AttnArgs &a, const MfmaPlan &plan, void *workspace, hipStream_t stream) {
    if (a.batch == 0 || a.max_nodes == 0) return hipSuccess;
    // bf16 calls with work always take the matrix-core kernel
    if (a.dtype != TV_F32) return hipErrorInvalidValue;
    Slices sl;
    if (plan.splits > 1) {
        sl.count = plan.splits;
        sl.keys = plan.keys_per_split;
        sl.ml = (float2 *)workspace;
        sl.o = (float *)((char *)workspace + align256((size_t)a.total_nodes * a.hq * sl.count * sizeof(float2)));
    }
    return a.head_dim == 64 ? launch_typed<float, 64>(a, sl, stream) : launch_typed<float, 128>(a, sl, stream);
}

}  // namespace tv
