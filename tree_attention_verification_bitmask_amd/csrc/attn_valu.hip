// tree_attn_verify, generic VALU path: one workgroup per (node, query head).
//
// [TSD] = "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
// Tree Attention Accelerate LLM Serving" (llms.blog), section "The Tree
// Attention Mechanism": each node attends to the whole prefix and to the tree
// nodes on its own root-to-node branch (parts 1 and 2).
//
// This path serves fp32 inputs (bf16 calls take the matrix-core kernel).
// The key axis is dealt over the workgroup's W wavefronts in chunks of 64
// keys (chunk c to wave c mod W), one key per lane: the lane
// computes its key's logit against q (held in LDS and read as a broadcast),
// the wave reduces max and sum (online softmax), and then every lane
// accumulates its own output channels over the 64 probabilities (shuffled
// from their lanes), reading V rows coalesced.  At the end the waves' (max,
// sum, output) are merged through LDS.  Tree keys j > i are never ancestors
// of node i (parents precede children), so the key loop stops at P + i + 1.
// All arithmetic is fp32; exp is expf.
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
template <>
struct Elem<uint16_t> {
    static __device__ __forceinline__ float ld(const uint16_t *p, int64_t i) {
        return __uint_as_float((uint32_t)p[i] << 16);
    }
    static __device__ __forceinline__ void st(uint16_t *p, int64_t i, float x) {
        p[i] = (uint16_t)(pack_bf16x2(x, 0.f) & 0xFFFFu);
    }
};

// 8 consecutive elements of a row starting at element e (16-byte aligned for
// bf16, 32 bytes read for fp32) -> fp32.
template <typename T>
__device__ __forceinline__ void load8(const T *row, int e, float out[8]);
template <>
__device__ __forceinline__ void load8<float>(const float *row, int e, float out[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(row + e);
    const float4 c = *reinterpret_cast<const float4 *>(row + e + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = c.x; out[5] = c.y; out[6] = c.z; out[7] = c.w;
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *row, int e, float out[8]) {
    const uint4 a = *reinterpret_cast<const uint4 *>(row + e);
    out[0] = bf16_lo(a.x); out[1] = bf16_hi(a.x);
    out[2] = bf16_lo(a.y); out[3] = bf16_hi(a.y);
    out[4] = bf16_lo(a.z); out[5] = bf16_hi(a.z);
    out[6] = bf16_lo(a.w); out[7] = bf16_hi(a.w);
}

template <typename T, int D, int W>
__global__ void __launch_bounds__(64 * W) attn_valu_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const int32_t *__restrict__ cu_nodes, const int32_t *__restrict__ kv_start,
    const int32_t *__restrict__ prefix_len, const uint64_t *__restrict__ anc, int total_nodes,
    int max_nodes, int max_prefix, int64_t kv_rows, int hq, int hkv, float scale, T *__restrict__ out,
    int32_t *__restrict__ err, const int32_t *__restrict__ table, int64_t table_stride,
    const float2 *__restrict__ rope_cs) {
    constexpr int CPL = D / 64;  // output channels per lane
    __shared__ float qs[D];
    __shared__ float wm[W], wl[W];
    __shared__ float wacc[W][D];
    const int i = blockIdx.x;   // request-local node
    const int h = blockIdx.y;   // query head
    const int b = blockIdx.z;   // request
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int lo;
    const int n = request_nodes(cu_nodes, b, total_nodes, max_nodes, &lo);
    const int P = prefix_len[b];
    const int64_t ks = table ? 0 : kv_start[b];
    const bool rows_bad = table ? ((int64_t)P + n > table_stride) : (ks < 0 || ks + P + n > kv_rows);
    if (n < 0 || P < 0 || P > max_prefix || rows_bad) {
        if (i == 0 && h == 0 && tid == 0) report(err, TV_DEVERR_BAD_REQUEST, b);
        return;
    }
    if (i >= n) return;
    const int G = hq / hkv;
    const int g = h / G;
    const int words = (max_nodes + 63) / 64;
    const int64_t t = (int64_t)lo + i;
    const uint64_t *arow = anc + t * words;

    if (rope_cs) {
        // channel e paired with e + D/2, rotated in fp32 by the node's angle
        for (int e = tid; e < D / 2; e += 64 * W) {
            const float x1 = Elem<T>::ld(q, (t * hq + h) * D + e);
            const float x2 = Elem<T>::ld(q, (t * hq + h) * D + e + D / 2);
            const float2 cs = rope_cs[t * (D / 2) + e];
            qs[e] = x1 * cs.x - x2 * cs.y;
            qs[e + D / 2] = x2 * cs.x + x1 * cs.y;
        }
    } else {
        for (int e = tid; e < D; e += 64 * W) qs[e] = Elem<T>::ld(q, (t * hq + h) * D + e);
    }
    __syncthreads();

    const int64_t kv_stride = (int64_t)hkv * D;  // elements per cache row
    const T *kbase = k + (int64_t)g * D;
    const T *vbase = v + (int64_t)g * D;
    const int32_t *trow = table ? table + (int64_t)b * table_stride : nullptr;
    const int nkeys = P + i + 1;

    float m = -INFINITY, l = 0.f;
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;

    for (int c0 = 64 * wv; c0 < nkeys; c0 += 64 * W) {
        const int key = c0 + lane;
        bool ok = key < nkeys;
        if (ok && key >= P) {
            const int j = key - P;
            ok = (arow[j >> 6] >> (j & 63)) & 1ull;
        }
        // cache row of this lane's key (key u's row is read from lane u below)
        int64_t krow = ks + key;
        if (trow && key < nkeys) {
            krow = trow[key];
            if (krow < 0 || krow >= kv_rows) {
                report(err, TV_DEVERR_BAD_SLOT, b);
                krow = 0;
            }
        }
        float s = -INFINITY;
        if (ok) {
            const T *kr = kbase + krow * kv_stride;
            float dot = 0.f;
#pragma unroll 4
            for (int e = 0; e < D; e += 8) {
                float kk[8];
                load8<T>(kr, e, kk);
#pragma unroll
                for (int u = 0; u < 8; ++u) dot = fmaf(qs[e + u], kk[u], dot);
            }
            s = dot * scale;
        }
        const float mc = wave_max(s);
        const float mn = fmaxf(m, mc);
        // A chunk can be fully masked (P == 0 and none of its nodes is an
        // ancestor); while no finite logit has been seen, use 0 as the
        // reference so that nothing evaluates exp(-inf - -inf).
        const float mref = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = expf(m - mref);
        const float p = ok ? expf(s - mref) : 0.f;
        l = l * alpha + wave_sum(p);
        m = mn;
        const int cnt = min(64, nkeys - c0);
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] *= alpha;
        for (int u = 0; u < cnt; ++u) {
            const float pu = __shfl(p, u, 64);
            if (pu == 0.f) continue;  // masked key (uniform branch)
            const T *vr = vbase + (int64_t)__shfl((long long)krow, u, 64) * kv_stride;
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] = fmaf(pu, Elem<T>::ld(vr, lane + 64 * c), acc[c]);
        }
    }
    // merge the waves: M = max m_w, out = sum_w e^(m_w - M) acc_w / sum_w e^(m_w - M) l_w
    // (a wave that saw no key, or only masked ones, has l = 0 and adds nothing)
    if (lane == 0) {
        wm[wv] = m;
        wl[wv] = l;
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) wacc[wv][lane + 64 * c] = acc[c];
    __syncthreads();
    if (tid < D) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, wm[w]);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            if (wl[w] > 0.f) {
                const float a = expf(wm[w] - M);
                L = fmaf(a, wl[w], L);
                o = fmaf(a, wacc[w][tid], o);
            }
        }
        Elem<T>::st(out, (t * hq + h) * D + tid, o / L);
    }
}

// Eight waves per workgroup; sixteen when the key axis is long (then the
// workgroups are few for a small tree and each needs more keys in flight).
// Measured, fp32, Hq 32 / Hkv 8, d 128 (us per call, 8 against 16 waves): one
// node over 8192 keys 475 / 295; 64 nodes over 1024 keys 290 / 319; 16 nodes
// over 128 keys 23 / 38.
template <typename T, int D, int W>
hipError_t launch_waves(const AttnArgs &a, hipStream_t stream) {
    dim3 grid(a.max_nodes, a.hq, a.batch);
    hipLaunchKernelGGL((attn_valu_kernel<T, D, W>), grid, dim3(64 * W), 0, stream, (const T *)a.q,
                       (const T *)a.k, (const T *)a.v, a.cu_nodes, a.kv_start, a.prefix_len, a.anc,
                       a.total_nodes, a.max_nodes, a.max_prefix, a.kv_rows, a.hq, a.hkv, a.scale,
                       (T *)a.out, a.err, a.table, a.table_stride, a.rope_cs);
    return hipGetLastError();
}
template <typename T, int D>
hipError_t launch_typed(const AttnArgs &a, hipStream_t stream) {
    return (int64_t)a.max_prefix + a.max_nodes >= 4096 ? launch_waves<T, D, 16>(a, stream)
                                                       : launch_waves<T, D, 8>(a, stream);
}

}  // namespace

hipError_t launch_attn_valu(const AttnArgs &a, hipStream_t stream) {
    if (a.batch == 0 || a.max_nodes == 0) return hipSuccess;
    if (a.dtype == TV_F32) {
        return a.head_dim == 64 ? launch_typed<float, 64>(a, stream) : launch_typed<float, 128>(a, stream);
    }
    return a.head_dim == 64 ? launch_typed<uint16_t, 64>(a, stream)
                            : launch_typed<uint16_t, 128>(a, stream);
}

}  // namespace tv
