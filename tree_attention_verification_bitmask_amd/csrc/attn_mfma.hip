// tree_attn_verify, MFMA path (bf16 in, fp32 accumulate) for gfx950.
//
// [TSD] = "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
// Tree Attention Accelerate LLM Serving" (llms.blog), section "The Tree
// Attention Mechanism": every node of the flattened tree attends to the whole
// prefix KV cache plus its own ancestors-or-self (parts 1 and 2).
//
// Rows and tiles.  For one request b and KV head g the query rows are the
// (node, head-in-group) pairs r = node * G + j, G = hq / hkv: the G heads
// sharing a KV head are stacked so that one K/V stream serves N*G rows.  A
// workgroup of 4 wavefronts takes 128 rows (32 per wave) and one slice of the
// key axis; K/V are staged 64 keys at a time through LDS and read by all four
// waves.
//
// Transposed products.  Each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 channels from LDS, B = 16
// channels x 32 query rows from registers).  The LDS row a lane reads is
// permuted (slot_of_key) so that in the 32x32 accumulator each lane holds one
// query row and 16 *consecutive* keys: softmax max/sum need one exchange
// between the two 32-lane halves (v_permlane32_swap) and nothing else.  Then
// O^T += V^T P^T with A = V^T (32 channels x 16 keys, from a transposed LDS
// copy of V) and B = P^T, which is exactly the probabilities the lane already
// holds, converted to bf16 -- no data movement between the two products.  The
// O^T accumulator again gives each lane one query row, so the online-softmax
// rescale is lane-local.
//
// The ancestor mask is applied per lane: the lane extracts the 16 bits of its
// node's packed row that cover its 16 keys (prefix keys are always allowed,
// keys past the slice end never) and sets the logits of cleared bits to -inf.
//
// Split key axis.  The host picks `splits` slices of `keys_per_split` keys
// (multiples of 64) so that the grid fills the chip.  With one slice the
// kernel writes the normalised bf16 output; otherwise it writes fp32 partials
// (unnormalised O, running max m, sum l) and attn_combine_kernel merges them.
//
// XCD-aware order.  Workgroup ids are dealt round-robin to the 8 XCDs; the
// kernel maps id -> task so that each XCD gets a contiguous block of tasks,
// and tasks are ordered with the row tiles of one (request, KV head, slice)
// adjacent, so the tiles that read the same K/V run on one XCD and share its
// L2.
#include "tv_device.h"
#include "tv_launch.h"

#include <stdlib.h>

namespace tv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileRows = 32 * kWaves;  // query rows per workgroup
constexpr int kChunk = 64;              // keys per LDS stage
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Smem {
    static constexpr int kStride = D + 8;       // bf16 per K row (pad: 16 B)
    static constexpr int vStride = kChunk + 8;  // bf16 per V^T row (pad: 16 B)
    uint16_t k[kChunk * kStride];
    uint16_t vt[D * vStride];
};

// Physical key p (0..31) of a 32-key block is stored at LDS row slot_of_key(p)
// so that accumulator row 8*(i/4) + 4*half + (i%4) of lane (col, half) is key
// 16*half + i.
__device__ __forceinline__ int slot_of_key(int p) {
    return 8 * ((p >> 2) & 3) + 4 * (p >> 4) + (p & 3);
}

__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Bits e = 0..15 set iff key (key0 + e) is visible to the node whose packed
// ancestor row is `arow`: prefix keys (< P) always, tree key P + j iff bit j,
// nothing at or past `key_hi`.
__device__ __forceinline__ uint32_t visible16(const uint64_t *__restrict__ arow, int words, int key0,
                                              int P, int key_hi) {
    uint32_t bits;
    const int j0 = key0 - P;
    if (j0 <= -16) {
        bits = 0xFFFFu;
    } else if (j0 < 0) {
        const int pre = -j0;  // 1..15 prefix keys, then tree nodes 0..
        bits = ((uint32_t)(arow[0] << pre) & 0xFFFFu) | ((1u << pre) - 1u);
    } else {
        const int w = j0 >> 6, sh = j0 & 63;
        if (w >= words) {
            bits = 0;
        } else {
            const uint64_t lo = arow[w];
            const uint64_t hi = (sh > 48 && w + 1 < words) ? arow[w + 1] : 0ull;
            const uint64_t x = sh ? ((lo >> sh) | (hi << (64 - sh))) : lo;
            bits = (uint32_t)x & 0xFFFFu;
        }
    }
    const int nvalid = key_hi - key0;
    if (nvalid < 16) bits &= nvalid <= 0 ? 0u : ((1u << nvalid) - 1u);
    return bits;
}

struct KParams {
    const uint16_t *q, *k, *v;
    const int32_t *cu_nodes, *kv_start, *prefix_len;
    const uint64_t *anc;
    int batch, total_nodes, max_nodes, max_prefix;
    int64_t kv_rows;
    int hq, hkv, words;
    int row_tiles, splits, keys_per_split;
    float c;  // scale * log2(e)
    uint16_t *out;
    float *ws_o;   // [tiles][splits][128][D]
    float2 *ws_ml; // [tiles][splits][128]
    int32_t *err;
};

template <int D>
__global__ void __launch_bounds__(kThreads) attn_mfma_kernel(KParams p) {
    constexpr int KV16 = D / 8;                     // 16-byte chunks per K/V row
    constexpr int KLOADS = kChunk * KV16 / kThreads; // K vectors per thread per chunk
    constexpr int DB = D / 32;                      // 32-channel blocks of O
    constexpr int KS = D / 16;                      // k-steps of Q K^T
    __shared__ Smem<D> sm;

    // ---- task decode (XCD-aware) -------------------------------------------
    const int ntasks = p.batch * p.hkv * p.splits * p.row_tiles;
    const int per_xcd = (ntasks + kXcds - 1) / kXcds;
    const int wid = blockIdx.x;
    const int task = (wid % kXcds) * per_xcd + wid / kXcds;
    if (task >= ntasks) return;
    const int rt = task % p.row_tiles;
    int rest = task / p.row_tiles;
    const int s = rest % p.splits;
    rest /= p.splits;
    const int g = rest % p.hkv;
    const int b = rest / p.hkv;

    int lo;
    const int n = request_nodes(p.cu_nodes, b, p.total_nodes, p.max_nodes, &lo);
    const int P = p.prefix_len[b];
    const int64_t ks = p.kv_start[b];
    if (n < 0 || P < 0 || P > p.max_prefix || ks < 0 || ks + P + n > p.kv_rows) {
        if (g == 0 && rt == 0 && s == 0 && threadIdx.x == 0) report(p.err, TV_DEVERR_BAD_REQUEST, b);
        return;
    }
    const int G = p.hq / p.hkv;
    const int rows_b = n * G;
    const int row0 = rt * kTileRows;
    if (row0 >= rows_b) return;
    const int row_end = min(rows_b, row0 + kTileRows);
    const int key_end = P + (row_end - 1) / G + 1;  // tree keys past the tile's last node are never visible
    const int k_lo = s * p.keys_per_split;
    if (k_lo >= key_end) return;
    const int k_hi = min(k_lo + p.keys_per_split, key_end);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 31;  // query row within the wave
    const int half = lane >> 5;

    // ---- this lane's query row ---------------------------------------------
    const int r = row0 + wave * 32 + col;
    const bool row_ok = r < row_end;
    const int node = row_ok ? r / G : (row_end - 1) / G;
    const int head = g * G + (row_ok ? r % G : 0);
    const int64_t t = (int64_t)lo + node;
    const uint64_t *arow = p.anc + t * p.words;
    bf16x8_t qb[KS];
    {
        const uint16_t *qrow = p.q + (t * p.hq + head) * D + 8 * half;
#pragma unroll
        for (int k16 = 0; k16 < KS; ++k16) {
            uint4 x = *reinterpret_cast<const uint4 *>(qrow + 16 * k16);
            if (!row_ok) x = make_uint4(0, 0, 0, 0);
            qb[k16] = __builtin_bit_cast(bf16x8_t, x);
        }
    }

    const int64_t kv_stride = (int64_t)p.hkv * D;  // elements per cache row
    const uint16_t *kbase = p.k + ks * kv_stride + (int64_t)g * D;
    const uint16_t *vbase = p.v + ks * kv_stride + (int64_t)g * D;

    // ---- global -> register staging of one 64-key chunk --------------------
    uint4 kreg[KLOADS];
    uint4 vreg[4];
    const int vkg = tid & 15;  // V: key group (4 keys) ...
    const int vdc = tid >> 4;  // ... and 8-channel column chunk
    auto fetch = [&](int c0) {
#pragma unroll
        for (int u = 0; u < KLOADS; ++u) {
            const int e = u * kThreads + tid;
            const int row = e / KV16, c16 = e % KV16;
            const int key = c0 + row;
            kreg[u] = key < k_hi ? *reinterpret_cast<const uint4 *>(kbase + (int64_t)key * kv_stride + c16 * 8)
                                 : make_uint4(0, 0, 0, 0);
        }
        if (vdc < KV16) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int key = c0 + 4 * vkg + rr;
                vreg[rr] = key < k_hi
                               ? *reinterpret_cast<const uint4 *>(vbase + (int64_t)key * kv_stride + vdc * 8)
                               : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int u = 0; u < KLOADS; ++u) {
            const int e = u * kThreads + tid;
            const int row = e / KV16, c16 = e % KV16;
            const int lrow = (row & ~31) + slot_of_key(row & 31);
            *reinterpret_cast<uint4 *>(&sm.k[lrow * Smem<D>::kStride + c16 * 8]) = kreg[u];
        }
        if (vdc < KV16) {
            const uint32_t a0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
            const uint32_t a1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
            const uint32_t a2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
            const uint32_t a3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
            for (int m2 = 0; m2 < 4; ++m2) {
                // channels 2*m2 (low halves) and 2*m2+1 (high halves) of 4 keys
                const uint32_t e01 = __builtin_amdgcn_perm(a1[m2], a0[m2], 0x05040100u);
                const uint32_t e23 = __builtin_amdgcn_perm(a3[m2], a2[m2], 0x05040100u);
                const uint32_t o01 = __builtin_amdgcn_perm(a1[m2], a0[m2], 0x07060302u);
                const uint32_t o23 = __builtin_amdgcn_perm(a3[m2], a2[m2], 0x07060302u);
                const int d = vdc * 8 + 2 * m2;
                *reinterpret_cast<uint2 *>(&sm.vt[d * Smem<D>::vStride + 4 * vkg]) = make_uint2(e01, e23);
                *reinterpret_cast<uint2 *>(&sm.vt[(d + 1) * Smem<D>::vStride + 4 * vkg]) = make_uint2(o01, o23);
            }
        }
    };

    // ---- main loop ------------------------------------------------------------
    f32x16_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float c = p.c;

    fetch(k_lo);
    for (int c0 = k_lo; c0 < k_hi; c0 += kChunk) {
        __syncthreads();  // everyone is done reading the previous chunk
        stash();
        __syncthreads();
        if (c0 + kChunk < k_hi) fetch(c0 + kChunk);  // in flight during the math below

        f32x16_t sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
            const uint16_t *arow_lds = &sm.k[(kb * 32 + col) * Smem<D>::kStride + 8 * half];
#pragma unroll
            for (int k16 = 0; k16 < KS; ++k16) {
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(arow_lds + 16 * k16));
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[k16], sacc[kb], 0, 0, 0);
            }
            const uint32_t vis = visible16(arow, p.words, c0 + kb * 32 + 16 * half, P, k_hi);
            if (vis != 0xFFFFu) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (!((vis >> i) & 1u)) sacc[kb][i] = -INFINITY;
            }
        }
        // online softmax over this chunk's 64 keys (32 per lane half)
        float mloc = sacc[0][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mloc = fmaxf(mloc, sacc[0][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, sacc[1][i]);
        mloc = halves_max(mloc);
        const float mn = fmaxf(m, mloc);
        const float mref = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = __builtin_amdgcn_exp2f((m - mref) * c);
        const float nb = -mref * c;
        float psum = 0.f;
        bf16x8_t pb[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                uint32_t w[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * tt + 2 * j], c, nb));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * tt + 2 * j + 1], c, nb));
                    psum += p0 + p1;
                    w[j] = pack_bf16x2(p0, p1);
                }
                pb[kb][tt] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
            }
        }
        l = l * alpha + psum;
        m = mn;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint16_t *vrow = &sm.vt[(db * 32 + col) * Smem<D>::vStride + kb * 32 + 16 * half + 8 * tt];
                    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(vrow));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][tt], oacc[db], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue -------------------------------------------------------------
    const float ltot = halves_sum(l);
    if (!row_ok) return;
    if (p.splits == 1) {
        const float inv = 1.f / ltot;
        uint16_t *orow = p.out + (t * p.hq + head) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d = db * 32 + 8 * i4 + 4 * half;
                const uint32_t w0 = pack_bf16x2(oacc[db][4 * i4 + 0] * inv, oacc[db][4 * i4 + 1] * inv);
                const uint32_t w1 = pack_bf16x2(oacc[db][4 * i4 + 2] * inv, oacc[db][4 * i4 + 3] * inv);
                *reinterpret_cast<uint2 *>(orow + d) = make_uint2(w0, w1);
            }
    } else {
        const int tile = (b * p.hkv + g) * p.row_tiles + rt;
        const int64_t prow = ((int64_t)tile * p.splits + s) * kTileRows + wave * 32 + col;
        float *orow = p.ws_o + prow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d = db * 32 + 8 * i4 + 4 * half;
                *reinterpret_cast<float4 *>(orow + d) =
                    make_float4(oacc[db][4 * i4 + 0], oacc[db][4 * i4 + 1], oacc[db][4 * i4 + 2], oacc[db][4 * i4 + 3]);
            }
        if (half == 0) p.ws_ml[prow] = make_float2(m, ltot);
    }
}

// Merge the per-slice partials of one row tile: O = sum_s w_s O_s / sum_s w_s l_s
// with w_s = 2^((m_s - M) c), M = max_s m_s.
template <int D>
__global__ void __launch_bounds__(kThreads) attn_combine_kernel(KParams p) {
    constexpr int TPR = D / 4;              // threads per row (4 channels each)
    constexpr int RPB = kThreads / TPR;     // rows per block
    const int tile = blockIdx.x;
    const int rt = tile % p.row_tiles;
    const int g = (tile / p.row_tiles) % p.hkv;
    const int b = tile / (p.row_tiles * p.hkv);
    int lo;
    const int n = request_nodes(p.cu_nodes, b, p.total_nodes, p.max_nodes, &lo);
    const int P = p.prefix_len[b];
    const int64_t ks = p.kv_start[b];
    if (n < 0 || P < 0 || P > p.max_prefix || ks < 0 || ks + P + n > p.kv_rows) return;
    const int G = p.hq / p.hkv;
    const int rows_b = n * G;
    const int row0 = rt * kTileRows;
    if (row0 >= rows_b) return;
    const int row_end = min(rows_b, row0 + kTileRows);
    const int key_end = P + (row_end - 1) / G + 1;
    const int nsplit = min(p.splits, (key_end + p.keys_per_split - 1) / p.keys_per_split);
    const int lrow = blockIdx.y * RPB + threadIdx.x / TPR;
    const int r = row0 + lrow;
    if (lrow >= kTileRows || r >= row_end) return;
    const int d = (threadIdx.x % TPR) * 4;
    const int64_t base = (int64_t)tile * p.splits * kTileRows + lrow;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, p.ws_ml[base + (int64_t)s * kTileRows].x);
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < nsplit; ++s) {
        const int64_t pr = base + (int64_t)s * kTileRows;
        const float2 ml = p.ws_ml[pr];
        if (ml.x == -INFINITY) continue;
        const float w = __builtin_amdgcn_exp2f((ml.x - M) * p.c);
        const float4 o = *reinterpret_cast<const float4 *>(p.ws_o + pr * D + d);
        L = fmaf(w, ml.y, L);
        acc.x = fmaf(w, o.x, acc.x);
        acc.y = fmaf(w, o.y, acc.y);
        acc.z = fmaf(w, o.z, acc.z);
        acc.w = fmaf(w, o.w, acc.w);
    }
    const float inv = 1.f / L;
    const int node = r / G;
    const int head = g * G + r % G;
    uint16_t *orow = p.out + (((int64_t)lo + node) * p.hq + head) * D;
    *reinterpret_cast<uint2 *>(orow + d) =
        make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
}

int env_int(const char *name, int dflt) {
    const char *s = getenv(name);
    if (!s || !*s) return dflt;
    return atoi(s);
}

}  // namespace

MfmaPlan plan_attn_mfma(int batch, int total_nodes, int max_nodes, int max_prefix, int hq, int hkv,
                        int head_dim, tv_dtype dtype) {
    (void)total_nodes;
    MfmaPlan plan;
    const int G = hkv > 0 ? hq / hkv : 0;
    // MFMA only where (nodes x GQA group) fills at least one 32-row tile
    if (dtype != TV_BF16 || (head_dim != 64 && head_dim != 128) || batch <= 0 || max_nodes * G < 32)
        return plan;
    plan.use = true;
    plan.rows_per_tile = kTileRows;
    plan.row_tiles = (max_nodes * G + kTileRows - 1) / kTileRows;
    const int span = max_prefix + max_nodes;                 // longest key axis
    const int chunks = (span + kChunk - 1) / kChunk;
    const long base_tasks = (long)batch * hkv * plan.row_tiles;
    // Fill the chip: aim for about two workgroups per CU (256 CUs).  A tuning
    // override (TV_MFMA_SPLITS) may fix the count instead.
    const long target = 512;
    int splits = (int)((target + base_tasks - 1) / base_tasks);
    splits = env_int("TV_MFMA_SPLITS", splits);
    if (splits < 1) splits = 1;
    if (splits > chunks) splits = chunks;
    const int cps = (chunks + splits - 1) / splits;         // chunks per split
    plan.keys_per_split = cps * kChunk;
    plan.splits = (chunks + cps - 1) / cps;
    if (plan.splits > 1) {
        const size_t rows = (size_t)base_tasks * plan.splits * kTileRows;
        plan.ws_bytes = rows * head_dim * sizeof(float);
        plan.ws_bytes = (plan.ws_bytes + 255) & ~(size_t)255;
        plan.ws_bytes += rows * sizeof(float2);
    }
    return plan;
}

hipError_t launch_attn_mfma(const AttnArgs &a, const MfmaPlan &plan, void *workspace, hipStream_t stream) {
    KParams p;
    p.q = (const uint16_t *)a.q;
    p.k = (const uint16_t *)a.k;
    p.v = (const uint16_t *)a.v;
    p.cu_nodes = a.cu_nodes;
    p.kv_start = a.kv_start;
    p.prefix_len = a.prefix_len;
    p.anc = a.anc;
    p.batch = a.batch;
    p.total_nodes = a.total_nodes;
    p.max_nodes = a.max_nodes;
    p.max_prefix = a.max_prefix;
    p.kv_rows = a.kv_rows;
    p.hq = a.hq;
    p.hkv = a.hkv;
    p.words = (a.max_nodes + 63) / 64;
    p.row_tiles = plan.row_tiles;
    p.splits = plan.splits;
    p.keys_per_split = plan.keys_per_split;
    p.c = a.scale * kLog2e;
    p.out = (uint16_t *)a.out;
    p.err = a.err;
    p.ws_o = nullptr;
    p.ws_ml = nullptr;
    if (plan.splits > 1) {
        const size_t rows = (size_t)a.batch * a.hkv * plan.row_tiles * plan.splits * kTileRows;
        size_t off = rows * a.head_dim * sizeof(float);
        off = (off + 255) & ~(size_t)255;
        p.ws_o = (float *)workspace;
        p.ws_ml = (float2 *)((char *)workspace + off);
    }
    const long ntasks = (long)a.batch * a.hkv * plan.splits * plan.row_tiles;
    const long grid = ((ntasks + kXcds - 1) / kXcds) * kXcds;
    const long tiles = (long)a.batch * a.hkv * plan.row_tiles;
    if (a.head_dim == 128) {
        hipLaunchKernelGGL(attn_mfma_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, p);
        if (plan.splits > 1)
            hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(tiles, kTileRows / (kThreads / 32)), dim3(kThreads), 0,
                               stream, p);
    } else {
        hipLaunchKernelGGL(attn_mfma_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, p);
        if (plan.splits > 1)
            hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(tiles, kTileRows / (kThreads / 16)), dim3(kThreads), 0,
                               stream, p);
    }
    return hipGetLastError();
}

}  // namespace tv
