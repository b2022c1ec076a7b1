// tree_target_sample: the target's sampled choice at every node (T > 0).
//
// [DT] = "DominoTree: Conditional Tree-Structured Drafting with Domino for
// Speculative Decoding", section 4.1: at temperature T > 0 the target token at
// each node is sampled while the draft stays deterministic.  [TSD] = "Tree-
// Structured Speculative Decoding ..." (llms.blog), "Verification and
// Acceptance Algorithms": with a point-mass draft the min(1, p/q) test accepts
// a child exactly when the target's sample equals its token, so the sampled
// tokens feed the same tree walk as the greedy ones.
//
// Row r's token is drawn from softmax(logits[r] / T) by inverse transform with
// the caller's uniform u[r]: with y = x * (1/T) and M = max y, the token is the
// smallest index whose cumulative weight sum_{j<=i} exp(y_j - M) exceeds
// u * sum_j exp(y_j - M).  The weights, sums and the comparison are float64,
// so the decision is taken in the same precision as a float64 reference; only
// the order of the additions differs, which moves a cumulative sum by a few
// float64 ulps.
//
// Two launches, both streaming:
//  * chunk pass: one wavefront per 2048-logit chunk of a row, four per
//    workgroup.  It writes the chunk's maximum Mc, its weight sum
//    Sc = sum exp(y - Mc) and the first NaN / +inf index to the workspace.
//    Every logit is read once from HBM here.
//  * pick pass: one workgroup per row.  It combines the chunk summaries (the
//    row maximum M, chunk weights Sc * exp(Mc - M) in chunk order), finds the
//    chunk where the running sum crosses u * S, and re-reads only that chunk
//    (2048 logits) to find the element.
// If rounding leaves no crossing (u * S >= S), the token is the last index with
// a positive weight.  Rows with a NaN give their first NaN, else rows with +inf
// their first +inf, and rows of -inf give 0.
#include "tv_device.h"
#include "tv_launch.h"
#include "exp64.h"

#include <limits.h>

namespace tv {
namespace {

constexpr int kSmpThreads = 256;
constexpr int kSmpWaves = kSmpThreads / 64;
constexpr int kSmpPer = 8;                          // consecutive logits per thread
constexpr int kSmpChunk = kSmpThreads * kSmpPer;    // logits per chunk

struct ChunkSum {
    double m;          // chunk maximum of y (-inf when every weight is zero)
    double s;          // sum over the chunk of exp(y - m)
    int32_t nan_first;  // first NaN index in the chunk, INT_MAX if none
    int32_t inf_first;  // first +inf index in the chunk, INT_MAX if none
};
static_assert(sizeof(ChunkSum) == 24, "chunk summary layout");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));


// The 8 logits of one thread at indices i0 .. i0+7 as float; indices at or
// past `vocab` read as -inf (weight zero, never NaN or +inf).
template <bool BF16>
__device__ __forceinline__ void load8(const char *rbase, int vocab, int i0, bool vec, float x[kSmpPer]) {
    if (vec && i0 + kSmpPer <= vocab) {
        if (BF16) {
            const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(rbase + (int64_t)i0 * 2));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[2 * q] = bf16_lo(w[q]);
                x[2 * q + 1] = bf16_hi(w[q]);
            }
        } else {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(rbase + (int64_t)i0 * 4);
            const u32x4 a = __builtin_nontemporal_load(p);
            const u32x4 b = __builtin_nontemporal_load(p + 1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[q] = __uint_as_float(a[q]);
                x[4 + q] = __uint_as_float(b[q]);
            }
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < kSmpPer; ++e) {
        const int i = i0 + e;
        if (i < vocab)
            x[e] = BF16 ? bf16_lo(reinterpret_cast<const uint16_t *>(rbase)[i])
                        : reinterpret_cast<const float *>(rbase)[i];
        else
            x[e] = -INFINITY;
    }
}

__device__ __forceinline__ double wave_max_d(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmax(x, __shfl_xor(x, off, 64));
    return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off, 64));
    return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off, 64));
    return x;
}

// Inclusive scan of one double per thread over the workgroup, in thread
// order; returns the thread's inclusive prefix, *total = the whole sum.
__device__ __forceinline__ double block_scan_d(double v, double *lds, double *total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    if (lane == 63) lds[wv] = v;
    __syncthreads();
    double before = 0.0, all = 0.0;
#pragma unroll
    for (int w = 0; w < kSmpWaves; ++w) {
        const double t = lds[w];
        if (w < wv) before += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + v;
}

// Chunk pass.  One wave per 2048-logit chunk, four chunks (of one row) per
// workgroup: every load of the chunk is issued up front (32 logits per lane,
// in 16-byte pieces, coalesced across the wave), the maximum and the sum are
// wave reductions, and the only barrier is the one that publishes the exp
// table.  The order of the additions within a chunk does not matter here;
// the pick pass scans elements in index order.
constexpr int kChunkWaves = 4;
constexpr int kLanePer = kSmpChunk / 64;  // logits per lane per chunk

template <bool BF16>
__global__ void __launch_bounds__(64 * kChunkWaves) sample_chunk_kernel(const void *__restrict__ logits, int vocab,
                                                                         int nchunks, double inv_t, ExpConst ek,
                                                                         ChunkSum *__restrict__ ws) {
    __shared__ double etab[kExpTable];
    constexpr int kEs = BF16 ? 2 : 4;
    constexpr int kPer16 = 16 / kEs;                 // logits per 16-byte piece
    constexpr int kPieces = kLanePer / kPer16;       // pieces per lane
    const int groups = (nchunks + kChunkWaves - 1) / kChunkWaves;
    const int row = (int)(blockIdx.x / groups);
    const int grp = (int)(blockIdx.x - (int64_t)row * groups);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int chunk = grp * kChunkWaves + wv;
    exp_table_fill(etab);
    __syncthreads();
    if (chunk >= nchunks) return;  // (wave-uniform; after the only barrier)
    const char *rbase = reinterpret_cast<const char *>(logits) + (int64_t)row * vocab * kEs;
    const bool vec = ((int64_t)vocab * kEs) % 16 == 0;
    const int c0 = chunk * kSmpChunk;
    // piece q of lane l covers logits c0 + (q * 64 + l) * kPer16 .. + kPer16 - 1
    float x[kLanePer];
    const bool full = vec && c0 + kSmpChunk <= vocab;
    if (full) {
        const u32x4 *vp = reinterpret_cast<const u32x4 *>(rbase + (int64_t)c0 * kEs);
        u32x4 w[kPieces];
#pragma unroll
        for (int q = 0; q < kPieces; ++q) w[q] = __builtin_nontemporal_load(vp + q * 64 + lane);
#pragma unroll
        for (int q = 0; q < kPieces; ++q)
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if (BF16) {
                    x[q * 8 + 2 * h] = bf16_lo(w[q][h]);
                    x[q * 8 + 2 * h + 1] = bf16_hi(w[q][h]);
                } else {
                    x[q * 4 + h] = __uint_as_float(w[q][h]);
                }
            }
    } else {
#pragma unroll
        for (int q = 0; q < kPieces; ++q)
#pragma unroll
            for (int e = 0; e < kPer16; ++e) {
                const int i = c0 + (q * 64 + lane) * kPer16 + e;
                x[q * kPer16 + e] = i < vocab ? (BF16 ? bf16_lo(reinterpret_cast<const uint16_t *>(rbase)[i])
                                                      : reinterpret_cast<const float *>(rbase)[i])
                                              : -INFINITY;
            }
    }
    // The maximum is taken on the logits themselves: x -> x * (1/T) rounds
    // monotonically (1/T > 0), so (double)max(x) * (1/T) is exactly max(y).
    // A NaN shows as a magnitude pattern above that of inf, a +inf as the
    // maximum; only a lane holding either scans its logits for the first of
    // each.
    float xm = -INFINITY;
    uint32_t amax = 0;
#pragma unroll
    for (int e = 0; e < kLanePer; ++e) {
        xm = fmaxf(xm, x[e]);  // ignores NaN
        amax = max(amax, __float_as_uint(x[e]) & 0x7FFFFFFFu);
    }
    int nan_i = INT_MAX, inf_i = INT_MAX;
    if (amax > 0x7F800000u || xm == INFINITY) {
#pragma unroll
        for (int q = kPieces - 1; q >= 0; --q)
#pragma unroll
            for (int e = kPer16 - 1; e >= 0; --e) {  // descending: the last write is the lane's first index
                const float v = x[q * kPer16 + e];
                const int i = c0 + (q * 64 + lane) * kPer16 + e;
                if (v != v) nan_i = i;
                if (v == INFINITY) inf_i = i;
            }
    }
    const double mc = wave_max_d((double)xm * inv_t);
    nan_i = wave_min_i(nan_i);
    inf_i = wave_min_i(inf_i);
    // weights relative to the chunk maximum (-inf and NaN logits give
    // y - mc = -inf or NaN, which exp_nonpos maps to 0); a chunk with +inf or
    // no finite logit has no meaningful sum: its row is decided by the
    // special indices
    double s = 0.0;
    if (mc > -INFINITY && mc < INFINITY) {
#pragma unroll
        for (int e = 0; e < kLanePer; ++e) s += exp_nonpos((double)x[e] * inv_t - mc, etab, ek);
    }
    s = wave_sum_d(s);
    if (lane == 0) {
        ChunkSum c;
        c.m = mc;
        c.s = (mc < INFINITY) ? s : 0.0;
        c.nan_first = nan_i;
        c.inf_first = inf_i;
        ws[(int64_t)row * nchunks + chunk] = c;
    }
}

// Weight of chunk c relative to the row maximum M.
__device__ __forceinline__ double chunk_weight(const ChunkSum &v, double M, const double *etab, const ExpConst &ek) {
    return v.m > -INFINITY ? v.s * exp_nonpos(v.m - M, etab, ek) : 0.0;
}

template <bool BF16>
__global__ void __launch_bounds__(kSmpThreads) sample_pick_kernel(const void *__restrict__ logits, int vocab,
                                                                   int nchunks, double inv_t, ExpConst ek,
                                                                   const double *__restrict__ u,
                                                                   const ChunkSum *__restrict__ ws,
                                                                   int32_t *__restrict__ token) {
    __shared__ double red_d[kSmpWaves];
    __shared__ int red_i[3][kSmpWaves];
    __shared__ double etab[kExpTable];
    constexpr int kEs = BF16 ? 2 : 4;
    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const ChunkSum *cs = ws + (int64_t)row * nchunks;
    const double ur = u[row];
    // the first tile of summaries stays in registers (all of them when the
    // row has at most 256 chunks, i.e. vocab <= 524288)
    ChunkSum v0;
    v0.m = -INFINITY;
    v0.s = 0.0;
    v0.nan_first = INT_MAX;
    v0.inf_first = INT_MAX;
    if (tid < nchunks) v0 = cs[tid];
    exp_table_fill(etab);

    // 1. row maximum and the special indices
    double m = v0.m;
    int nan_i = v0.nan_first, inf_i = v0.inf_first;
    for (int c = tid + kSmpThreads; c < nchunks; c += kSmpThreads) {
        const ChunkSum v = cs[c];
        m = fmax(m, v.m);
        nan_i = min(nan_i, v.nan_first);
        inf_i = min(inf_i, v.inf_first);
    }
    m = wave_max_d(m);
    nan_i = wave_min_i(nan_i);
    inf_i = wave_min_i(inf_i);
    if (lane == 0) {
        red_d[wv] = m;
        red_i[0][wv] = nan_i;
        red_i[1][wv] = inf_i;
    }
    __syncthreads();
    double M = red_d[0];
    nan_i = red_i[0][0];
    inf_i = red_i[1][0];
#pragma unroll
    for (int w = 1; w < kSmpWaves; ++w) {
        M = fmax(M, red_d[w]);
        nan_i = min(nan_i, red_i[0][w]);
        inf_i = min(inf_i, red_i[1][w]);
    }
    __syncthreads();
    if (nan_i != INT_MAX || inf_i != INT_MAX || !(M > -INFINITY)) {
        if (tid == 0) token[row] = nan_i != INT_MAX ? nan_i : (inf_i != INT_MAX ? inf_i : 0);
        return;
    }

    // 2. the chunk weights in chunk order: total S (the same block scans as
    // step 3, so the running sums there end exactly at S), and the last chunk
    // with a positive weight
    const int tiles = (nchunks + kSmpThreads - 1) / kSmpThreads;
    const double w0 = chunk_weight(v0, M, etab, ek);
    double tot0;
    const double incl0 = block_scan_d(w0, red_d, &tot0);
    double S = tot0;
    int last_pos = w0 > 0.0 ? tid : -1;
    for (int t = 1; t < tiles; ++t) {
        const int c = t * kSmpThreads + tid;
        const double w = c < nchunks ? chunk_weight(cs[c], M, etab, ek) : 0.0;
        if (w > 0.0) last_pos = c;
        double tot;
        block_scan_d(w, red_d, &tot);
        S += tot;
    }
    last_pos = wave_max_i(last_pos);
    if (lane == 0) red_i[2][wv] = last_pos;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kSmpWaves; ++w) last_pos = max(last_pos, red_i[2][w]);
    __syncthreads();

    // 3. the first chunk whose running sum exceeds u * S
    const double target = ur * S;
    double base = 0.0;  // running sum before the current tile
    int found = INT_MAX;
    double found_base = 0.0;
    for (int t = 0; t < tiles && found == INT_MAX; ++t) {
        const int c = t * kSmpThreads + tid;
        double w, incl, tot;
        if (t == 0) {
            w = w0;
            incl = incl0;
            tot = tot0;
        } else {
            w = c < nchunks ? chunk_weight(cs[c], M, etab, ek) : 0.0;
            incl = block_scan_d(w, red_d, &tot);
        }
        const int cand = (c < nchunks && base + incl > target) ? c : INT_MAX;
        const int wmin = wave_min_i(cand);
        if (lane == 0) red_i[0][wv] = wmin;
        // the lowest crossing thread of this wave leaves its exclusive base
        if (cand != INT_MAX && cand == wmin) red_d[wv] = base + (incl - w);
        __syncthreads();
        int best = INT_MAX, bw = -1;
#pragma unroll
        for (int w2 = 0; w2 < kSmpWaves; ++w2)
            if (red_i[0][w2] < best) {
                best = red_i[0][w2];
                bw = w2;
            }
        if (best != INT_MAX) {
            found = best;
            found_base = red_d[bw];
        }
        base += tot;
        __syncthreads();
    }
    // no crossing (u * S rounds to >= S, or u is not in [0, 1)): the last index
    // with a positive weight, found by an element scan that never crosses
    const bool fallback = found == INT_MAX;
    const int chunk = fallback ? max(last_pos, 0) : found;
    const double cbase = fallback ? 0.0 : found_base;
    const double ctarget = fallback ? INFINITY : target;

    // 4. the element: re-read the chunk, weights relative to the row maximum
    const char *rbase = reinterpret_cast<const char *>(logits) + (int64_t)row * vocab * kEs;
    const bool vec = ((int64_t)vocab * kEs) % 16 == 0;
    const int i0 = chunk * kSmpChunk + tid * kSmpPer;
    float x[kSmpPer];
    load8<BF16>(rbase, vocab, i0, vec, x);
    double w[kSmpPer];
    double own = 0.0;
    int last_i = -1;
#pragma unroll
    for (int e = 0; e < kSmpPer; ++e) {
        const double y = (double)x[e] * inv_t;
        w[e] = y > -INFINITY ? exp_nonpos(y - M, etab, ek) : 0.0;
        own += w[e];
        if (w[e] > 0.0) last_i = i0 + e;
    }
    double tot;
    const double incl = block_scan_d(own, red_d, &tot);
    double run = cbase + (incl - own);
    int cand = INT_MAX;
#pragma unroll
    for (int e = 0; e < kSmpPer; ++e) {
        run += w[e];
        if (cand == INT_MAX && run > ctarget) cand = i0 + e;
    }
    cand = wave_min_i(cand);
    last_i = wave_max_i(last_i);
    if (lane == 0) {
        red_i[0][wv] = cand;
        red_i[1][wv] = last_i;
    }
    __syncthreads();
    if (tid == 0) {
        int first = INT_MAX, last = -1;
#pragma unroll
        for (int w2 = 0; w2 < kSmpWaves; ++w2) {
            first = min(first, red_i[0][w2]);
            last = max(last, red_i[1][w2]);
        }
        // a chunk chosen by its positive weight holds an element with a
        // positive weight; the guard only keeps the index in range
        token[row] = first != INT_MAX ? first : (last >= 0 ? last : 0);
    }
}

}  // namespace

size_t target_sample_workspace(int rows, int vocab) {
    const int64_t nchunks = ((int64_t)vocab + kSmpChunk - 1) / kSmpChunk;
    return (size_t)rows * (size_t)nchunks * sizeof(ChunkSum);
}

int64_t target_sample_blocks(int rows, int vocab) {
    const int64_t nchunks = ((int64_t)vocab + kSmpChunk - 1) / kSmpChunk;
    return (int64_t)rows * nchunks;
}

hipError_t launch_target_sample(const void *logits, int rows, int vocab, tv_dtype dtype, double inv_t,
                                const double *u, int32_t *token, void *workspace, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const int nchunks = (int)(((int64_t)vocab + kSmpChunk - 1) / kSmpChunk);
    const unsigned blocks = (unsigned)((int64_t)rows * ((nchunks + kChunkWaves - 1) / kChunkWaves));
    ChunkSum *ws = reinterpret_cast<ChunkSum *>(workspace);
    const ExpConst ek = exp_const();
    if (dtype == TV_BF16) {
        hipLaunchKernelGGL(sample_chunk_kernel<true>, dim3(blocks), dim3(64 * kChunkWaves), 0, stream, logits, vocab,
                           nchunks, inv_t, ek, ws);
        hipLaunchKernelGGL(sample_pick_kernel<true>, dim3(rows), dim3(kSmpThreads), 0, stream, logits, vocab,
                           nchunks, inv_t, ek, u, ws, token);
    } else {
        hipLaunchKernelGGL(sample_chunk_kernel<false>, dim3(blocks), dim3(64 * kChunkWaves), 0, stream, logits, vocab,
                           nchunks, inv_t, ek, ws);
        hipLaunchKernelGGL(sample_pick_kernel<false>, dim3(rows), dim3(kSmpThreads), 0, stream, logits, vocab,
                           nchunks, inv_t, ek, u, ws, token);
    }
    return hipGetLastError();
}

}  // namespace tv
