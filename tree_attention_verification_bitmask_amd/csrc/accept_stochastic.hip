// tree_accept_stochastic: the tree walk at temperature T > 0 against a
// stochastic draft.
//
// [TSD] = "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
// Tree Attention Accelerate LLM Serving" (llms.blog), "Verification and
// Acceptance Algorithms", section "Exact Sampling Equivalence": a candidate x
// that the drafter proposed with probability q(x) is accepted with probability
// min(1, p(x) / q(x)), p the target's distribution; after a rejection a
// replacement comes from (p - q)+ normalised.  With several candidates at one
// node (the children, drawn from the same q) they are tried in ascending
// index, each against the residual left by the rejections before it.
//
// Two launches:
//  * chunk statistics: one wavefront per 2048-logit chunk of every row
//    (roots, then nodes), four per workgroup, writes the chunk's maximum m_c
//    of y = logit * (1/T) and s_c = sum exp(y - m_c), float64: every logit is
//    read once, by the whole GPU.
//  * walk: one workgroup of 1024 threads per request.  At each node it
//    merges that row's chunk statistics into M = max y and Z = sum exp(y - M)
//    (p(x) = exp(y_x - M) / Z).  A candidate's test reads p(x) and q(x) only.
//    The first rejection at a node writes the residual (p - q)+ to the
//    workspace and sums it in one pass; a later one takes two passes without
//    exponentials (the sum, then the residual).  The final draw: each thread
//    sums a contiguous range of weights in index order, a block scan gives
//    the range starts, and the range holding u * total is scanned again.
// All arithmetic is float64 (exp by the table-driven exp_nonpos), the
// precision of the acceptance decisions and of the draw; only the order of
// additions differs from a sequential sum.
#include "exp64.h"
#include "tv_device.h"
#include "tv_launch.h"

#include <limits.h>

namespace tv {
namespace {

constexpr int kStatWaves = 4;
constexpr int kStatChunk = 2048;  // logits per chunk statistic
constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / 64;

template <typename T>
__device__ __forceinline__ double ld64(const T *p, int64_t i);
template <>
__device__ __forceinline__ double ld64<float>(const float *p, int64_t i) { return (double)p[i]; }
template <>
__device__ __forceinline__ double ld64<uint16_t>(const uint16_t *p, int64_t i) {
    return (double)__uint_as_float((uint32_t)p[i] << 16);
}

__device__ __forceinline__ double wave_sum64(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
__device__ __forceinline__ double wave_max64(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmax(x, __shfl_xor(x, off, 64));
    return x;
}

// Block-wide sum / max over NW waves through `red` (NW doubles); every thread
// gets the result.
template <int NW>
__device__ __forceinline__ double block_sum64(double x, double *red) {
    x = wave_sum64(x);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wv] = x;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += red[w];
    return t;
}
template <int NW>
__device__ __forceinline__ double block_max64(double x, double *red) {
    x = wave_max64(x);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wv] = x;
    __syncthreads();
    double t = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) t = fmax(t, red[w]);
    return t;
}

// Chunk statistics: wave gw takes chunk gw % nchunks of row gw / nchunks.
template <typename T>
__global__ void __launch_bounds__(64 * kStatWaves) stoch_chunk_kernel(const T *__restrict__ root_logits,
                                                                      const T *__restrict__ node_logits, int batch,
                                                                      int rows, int vocab, int nchunks, double inv_t,
                                                                      ExpConst ek, double2 *__restrict__ cst) {
    __shared__ double etab[kExpTable];
    exp_table_fill(etab);
    __syncthreads();
    const int64_t gw = (int64_t)blockIdx.x * kStatWaves + (threadIdx.x >> 6);
    if (gw >= (int64_t)rows * nchunks) return;
    const int lane = threadIdx.x & 63;
    const int r = (int)(gw / nchunks), c = (int)(gw - (int64_t)r * nchunks);
    const T *row = r < batch ? root_logits + (int64_t)r * vocab : node_logits + (int64_t)(r - batch) * vocab;
    const int i0 = c * kStatChunk, i1 = min(vocab, i0 + kStatChunk);
    double y[kStatChunk / 64];
    double m = -INFINITY;
#pragma unroll
    for (int e = 0; e < kStatChunk / 64; ++e) {
        const int i = i0 + e * 64 + lane;
        y[e] = i < i1 ? ld64(row, i) * inv_t : -INFINITY;
        m = fmax(m, y[e]);
    }
    m = wave_max64(m);
    double sum = 0.0;
    if (m > -INFINITY) {
#pragma unroll
        for (int e = 0; e < kStatChunk / 64; ++e) sum += exp_nonpos(y[e] - m, etab, ek);
    }
    sum = wave_sum64(sum);
    if (lane == 0) cst[gw] = make_double2(m, sum);
}

template <typename T>
__global__ void __launch_bounds__(kWalkThreads) stoch_walk_kernel(
    const int32_t *__restrict__ parent, const int32_t *__restrict__ draft, const int32_t *__restrict__ cu_nodes,
    int batch, int total_nodes, int max_depth, const T *__restrict__ root_logits, const T *__restrict__ node_logits,
    int vocab, double inv_t, const float *__restrict__ root_q, const float *__restrict__ node_q,
    const double *__restrict__ u_accept, const double *__restrict__ u_final, const double2 *__restrict__ cst,
    int nchunks, ExpConst ek, double *__restrict__ res_all, int32_t *__restrict__ accept_len,
    int32_t *__restrict__ accept_idx, int32_t *__restrict__ next_token, int32_t *__restrict__ err) {
    __shared__ int kids[TV_MAX_NODES];
    __shared__ double etab[kExpTable];
    exp_table_fill(etab);  // (visible after the barrier of the checks below)
    __shared__ int wcount[kWalkWaves];
    __shared__ double red[kWalkWaves];
    __shared__ int sel[3];
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int32_t *idx_out = accept_idx + (int64_t)b * max_depth;
    for (int i = tid; i < max_depth; i += kWalkThreads) idx_out[i] = -1;

    // request checks: node range, parents, draft tokens
    int lo;
    const int n = request_nodes(cu_nodes, b, total_nodes, TV_MAX_NODES, &lo);
    if (n < 0) {
        if (tid == 0) {
            report(err, TV_DEVERR_BAD_REQUEST, b);
            accept_len[b] = 0;
            next_token[b] = -1;
        }
        return;
    }
    int bad = 0;
    if (tid < n) {
        const int pa = parent[lo + tid], d = draft[lo + tid];
        if (pa < -1 || pa >= tid) {
            report(err, TV_DEVERR_BAD_PARENT, lo + tid);
            bad = 1;
        }
        if (d >= vocab) {
            report(err, TV_DEVERR_BAD_TOKEN, lo + tid);
            bad = 1;
        }
    }
    if (__syncthreads_or(bad)) {
        if (tid == 0) {
            accept_len[b] = 0;
            next_token[b] = -1;
        }
        return;
    }

    double *res = res_all + (int64_t)b * vocab;
    int cur = -1, L = 0;
    bool implicit = true;  // the residual is still p itself
    double M = 0.0, Z = 1.0, S = 1.0;
    const T *lrow = nullptr;
    const float *qrow = nullptr;
    // r(v): the current residual (normalised)
    // (normalised by multiplying with 1/Z and 1/S: a float64 division costs
    // as much as the exponential, and these passes are float64-bound on one CU)
    double iZ = 1.0, iS = 1.0;
    auto p_at = [&](int v) { return exp_nonpos(ld64(lrow, v) * inv_t - M, etab, ek) * iZ; };
    auto r_at = [&](int v) { return implicit ? p_at(v) : res[v] * iS; };
    for (;;) {
        const int row = cur < 0 ? b : batch + lo + cur;
        lrow = cur < 0 ? root_logits + (int64_t)b * vocab : node_logits + (int64_t)(lo + cur) * vocab;
        qrow = cur < 0 ? root_q + (int64_t)b * vocab : node_q + (int64_t)(lo + cur) * vocab;
        // M and Z of the row from its chunk statistics (chunk order)
        {
            const double2 *rc = cst + (int64_t)row * nchunks;
            double mloc = -INFINITY;
            for (int c = tid; c < nchunks; c += kWalkThreads) mloc = fmax(mloc, rc[c].x);
            M = block_max64<kWalkWaves>(mloc, red);
            double part = 0.0;
            for (int c = tid; c < nchunks; c += kWalkThreads) {
                const double2 cs = rc[c];
                if (cs.x > -INFINITY) part += cs.y * exp_nonpos(cs.x - M, etab, ek);
            }
            Z = block_sum64<kWalkWaves>(part, red);
            iZ = 1.0 / Z;
        }
        implicit = true;
        // children of cur in ascending index (none once max_depth are accepted)
        const bool kid = L < max_depth && tid < n && parent[lo + tid] == cur;
        const uint64_t bal = __ballot(kid);
        if (lane == 0) wcount[wv] = __popcll(bal);
        __syncthreads();
        int before = 0, nk = 0;
#pragma unroll
        for (int w = 0; w < kWalkWaves; ++w) {
            before += w < wv ? wcount[w] : 0;
            nk += wcount[w];
        }
        if (kid) kids[before + __popcll(bal & ((1ull << lane) - 1ull))] = tid;
        __syncthreads();
        int acc = -1;
        for (int i = 0; i < nk; ++i) {  // uniform
            const int c = kids[i];
            const int x = draft[lo + c];
            if (x < 0) continue;  // dead leaf: not a candidate
            const double rx = r_at(x);
            const double qx = (double)qrow[x];
            const double a = qx > 0.0 ? fmin(1.0, rx / qx) : (rx > 0.0 ? 1.0 : 0.0);
            if (u_accept[lo + c] < a) {
                acc = c;
                break;
            }
            // rejected: r <- (r - q)+ / sum (r - q)+ (kept when that sum is 0)
            if (implicit) {
                // from p: one pass writes (p - q)+ and sums it; if the sum is
                // 0, r stays p (implicit) and the buffer is not read
                double s1 = 0.0;
#pragma unroll 8
                for (int v = tid; v < vocab; v += kWalkThreads) {
                    const double d = fmax(p_at(v) - (double)qrow[v], 0.0);
                    res[v] = d;
                    s1 += d;
                }
                s1 = block_sum64<kWalkWaves>(s1, red);
                if (s1 > 0.0) {
                    implicit = false;
                    S = s1;
                    iS = 1.0 / S;
                }
            } else {
                // from the stored residual: the sum first (the residual must
                // survive a zero sum), then the update in place
                double s1 = 0.0;
#pragma unroll 8
                for (int v = tid; v < vocab; v += kWalkThreads) s1 += fmax(res[v] * iS - (double)qrow[v], 0.0);
                s1 = block_sum64<kWalkWaves>(s1, red);
                if (s1 > 0.0) {
#pragma unroll 8
                    for (int v = tid; v < vocab; v += kWalkThreads) res[v] = fmax(res[v] * iS - (double)qrow[v], 0.0);
                    S = s1;
                    iS = 1.0 / S;
                    __syncthreads();
                }
            }
        }
        if (acc < 0) break;
        if (tid == 0) idx_out[L] = acc;
        ++L;
        cur = acc;
        __syncthreads();  // (kids is rebuilt for the next node)
    }

    // the next token: inverse transform over the residual's weights
    auto w_at = [&](int v) { return implicit ? exp_nonpos(ld64(lrow, v) * inv_t - M, etab, ek) : res[v]; };
    const int per = (vocab + kWalkThreads - 1) / kWalkThreads;
    const int v0 = min(vocab, tid * per), v1 = min(vocab, v0 + per);
    double local = 0.0;
    int last = -1;  // the range's last index with a positive weight
    // (this and the passes above are unrolled: their loads are independent,
    // so several are in flight at once instead of one memory round trip per
    // element)
#pragma unroll 8
    for (int v = v0; v < v1; ++v) {
        const double w = w_at(v);
        local += w;
        if (w > 0.0) last = v;
    }
    // exclusive block scan of the range sums (in thread order = index order)
    double incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    __syncthreads();
    if (lane == 63) red[wv] = incl;
    __syncthreads();
    double base = 0.0, total = 0.0;
#pragma unroll
    for (int w = 0; w < kWalkWaves; ++w) {
        base += w < wv ? red[w] : 0.0;
        total += red[w];
    }
    const double start = base + incl - local;
    const double thr = u_final[b] * total;
    if (tid == 0) {
        sel[0] = INT_MAX;  // the chosen index
        sel[1] = -1;       // the last index with a positive weight
        sel[2] = INT_MAX;  // the thread whose range holds thr
    }
    __syncthreads();
    // the range whose span holds thr (one, unless rounding makes two adjacent
    // spans overlap by an ulp: then the earlier range wins)
    if (local > 0.0 && start <= thr && thr < start + local) atomicMin(&sel[2], tid);
    // the last index with a positive weight, for a draw that rounding pushed
    // past the total
    if (last >= 0) atomicMax(&sel[1], last);
    __syncthreads();
    const int owner = sel[2];  // uniform
    if (owner != INT_MAX) {
        // That range scanned by the whole block (one weight per thread, an
        // inclusive block scan added to the range's start): the first index
        // whose running sum exceeds thr, else the range's last positive one.
        __shared__ double owner_start;
        __shared__ int owner_last;
        if (tid == owner) {
            owner_start = start;
            owner_last = last;
        }
        __syncthreads();
        const int r0 = min(vocab, owner * per), r1 = min(vocab, r0 + per);
        double run = owner_start;  // uniform: the running sum before the tile
        for (int t0 = r0; t0 < r1; t0 += kWalkThreads) {
            const bool in = t0 + tid < r1;
            const double w = in ? w_at(t0 + tid) : 0.0;
            double inc = w;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const double o = __shfl_up(inc, off, 64);
                if (lane >= off) inc += o;
            }
            __syncthreads();
            if (lane == 63) red[wv] = inc;
            __syncthreads();
            double before_w = 0.0, tile = 0.0;
#pragma unroll
            for (int w2 = 0; w2 < kWalkWaves; ++w2) {
                before_w += w2 < wv ? red[w2] : 0.0;
                tile += red[w2];
            }
            if (in && run + (before_w + inc) > thr) atomicMin(&sel[0], t0 + tid);
            __syncthreads();
            if (sel[0] != INT_MAX) break;  // uniform
            run += tile;
        }
        if (tid == 0 && sel[0] == INT_MAX) sel[0] = owner_last;
    }
    __syncthreads();
    if (tid == 0) {
        accept_len[b] = L;
        next_token[b] = owner != INT_MAX ? sel[0] : (sel[1] >= 0 ? sel[1] : 0);
    }
}

}  // namespace

size_t accept_stochastic_workspace(int batch, int total_nodes, int vocab) {
    const size_t nchunks = ((size_t)vocab + kStatChunk - 1) / kStatChunk;
    const size_t stats = (size_t)(batch + total_nodes) * nchunks * sizeof(double2);
    return ((stats + 255) & ~(size_t)255) + (size_t)batch * vocab * sizeof(double);
}

hipError_t launch_accept_stochastic(const int32_t *parent, const int32_t *draft, const int32_t *cu_nodes, int batch,
                                    int total_nodes, int max_depth, const void *root_logits,
                                    const void *node_logits, tv_dtype dtype, double inv_t, const float *root_q,
                                    const float *node_q, int vocab, const double *u_accept, const double *u_final,
                                    int32_t *accept_len, int32_t *accept_idx, int32_t *next_token, void *workspace,
                                    int32_t *err, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    const int nchunks = (vocab + kStatChunk - 1) / kStatChunk;
    const int rows = batch + total_nodes;
    double2 *cst = (double2 *)workspace;
    const size_t soff = ((size_t)rows * nchunks * sizeof(double2) + 255) & ~(size_t)255;
    double *res = (double *)((char *)workspace + soff);
    const ExpConst ek = exp_const();
    const unsigned blocks = (unsigned)(((int64_t)rows * nchunks + kStatWaves - 1) / kStatWaves);
    if (dtype == TV_BF16) {
        hipLaunchKernelGGL(stoch_chunk_kernel<uint16_t>, dim3(blocks), dim3(64 * kStatWaves), 0, stream,
                           (const uint16_t *)root_logits, (const uint16_t *)node_logits, batch, rows, vocab, nchunks,
                           inv_t, ek, cst);
        hipLaunchKernelGGL(stoch_walk_kernel<uint16_t>, dim3(batch), dim3(kWalkThreads), 0, stream, parent, draft,
                           cu_nodes, batch, total_nodes, max_depth, (const uint16_t *)root_logits,
                           (const uint16_t *)node_logits, vocab, inv_t, root_q, node_q, u_accept, u_final, cst,
                           nchunks, ek, res, accept_len, accept_idx, next_token, err);
    } else {
        hipLaunchKernelGGL(stoch_chunk_kernel<float>, dim3(blocks), dim3(64 * kStatWaves), 0, stream,
                           (const float *)root_logits, (const float *)node_logits, batch, rows, vocab, nchunks,
                           inv_t, ek, cst);
        hipLaunchKernelGGL(stoch_walk_kernel<float>, dim3(batch), dim3(kWalkThreads), 0, stream, parent, draft,
                           cu_nodes, batch, total_nodes, max_depth, (const float *)root_logits,
                           (const float *)node_logits, vocab, inv_t, root_q, node_q, u_accept, u_final, cst, nchunks,
                           ek, res, accept_len, accept_idx, next_token, err);
    }
    return hipGetLastError();
}

}  // namespace tv
