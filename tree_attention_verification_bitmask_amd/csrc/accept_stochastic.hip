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
// The residual after any number of rejections has a closed form.  If
// r = (p - c q)+ / W with W = sum (p - c q)+ (r = p is c = 0, W = 1), then
// (r - q)+ = (p - (c + W) q)+ / W, since W > 0 and q >= 0.  So the residual
// after the next rejection is (p - c' q)+ normalised, with c' = c + W (kept
// as it was if the new sum is 0).  A rejection costs one sum over the
// vocabulary, and a node's tests read that node's rows only: every node of
// every tree is decided at once, whether the walk reaches it or not, and the
// walk then follows the decisions.  The float64 passes over the vocabulary
// thus run on the whole GPU instead of on one workgroup walking a path.
//
// Launches, in stream order:
//  * front: two kinds of workgroups in one grid.  One per request (prep):
//    checks, each node's depth and its candidates (live children in
//    ascending index; none at depth max_depth) with what their tests read
//    (the token's logit and draft probability in the parent's rows, and the
//    uniform).  The others (stats), one wavefront per 2048-logit chunk of
//    every row (roots, then nodes): the chunk's maximum m_c of
//    y = logit * (1/T) and s_c = sum exp(y - m_c).  Every logit is read
//    once, by the whole GPU.
//  * pass j (j = 0 .. kLevels-1): one wavefront per (row, chunk).  Every
//    wavefront of an open row decides test j, all alike from the same
//    values; after a rejection each reads its chunk and adds up its share of
//    the next residual's sum.
//  * select: one workgroup per request: the walk along the decisions, then
//    the draw from the last node's residual by inverse transform (the chunk
//    weights scanned in chunk order, then the chosen chunk's elements in
//    index order).  A node on the path with more than kLevels candidates
//    continues its tests here, one workgroup-wide sum per rejection.
// All arithmetic is float64 (exp by the table-driven exp_nonpos), the
// precision of the acceptance decisions and of the draw; the residual is
// formed in the closed form above and the sums are added chunk by chunk, so
// only the rounding differs from a sequential update.
#include "exp64.h"
#include "tv_device.h"
#include "tv_launch.h"

#include <limits.h>

namespace tv {
namespace {

constexpr int kChunk = 2048;            // logits per chunk statistic / partial sum
constexpr int kPerLane = kChunk / 64;   // logits of one lane in a chunk
constexpr int kPassWaves = 4;           // chunks (wavefronts) per workgroup in the passes
constexpr int kLevels = 4;              // tests decided by whole-GPU passes; the rest in select
constexpr int kSlots = kLevels + 2;     // partial-sum slots: one per pass, two for select
constexpr int kFrontThreads = 1024;
constexpr int kFrontWaves = kFrontThreads / 64;
constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelPer = kChunk / kSelThreads;  // consecutive logits per thread in the element scan
static_assert(kFrontThreads >= TV_MAX_NODES && TV_MAX_NODES % 4 == 0, "one prep thread per node");

enum : int32_t { kClosed = 0, kOpen = 1 };
// dec[row]: the accepted child (global node index), or one of these
enum : int32_t { kDecFinal = -1, kDecContinue = -2 };

// One candidate: global node t with draft token x; y and q are the target's
// logit and the draft probability of x in the parent's rows; u its uniform.
struct Cand {
    int32_t t, x;
    float y, q;
    double u;
};
// What pass j-1 leaves for pass j about a row.  kOpen: test j-1 was rejected
// against the residual (c, W) of level `lev`, pass j-1 wrote the chunk sums
// of (p - c1 q)+ with c1 = c + W, and `next` is candidate j (if the row has
// one).  kClosed: the row needs nothing more.
struct Rec {
    int32_t status;
    int32_t lev;  // 0: r = p; s >= 1: r's chunk sums sit in slot s
    double c, W, c1;
    Cand next;
    int32_t pad[2];
};
// A node's residual once all its tests are rejected (or it has none).
struct Fin {
    double c, W;
    int32_t lev, pad;
};
static_assert(sizeof(Cand) == 24 && sizeof(Rec) == 64 && sizeof(Fin) == 24, "workspace records");

// Workspace segments, each 256-byte aligned.
struct Layout {
    size_t st, part, mz, rec, fin, kc, dec, c0, cand, bad, total;
};
Layout layout(int batch, int total_nodes, int vocab) {
    const size_t nch = ((size_t)vocab + kChunk - 1) / kChunk;
    const size_t rows = (size_t)batch + (size_t)total_nodes;
    Layout l;
    size_t off = 0;
    auto seg = [&](size_t bytes) {
        const size_t at = (off + 255) & ~(size_t)255;
        off = at + bytes;
        return at;
    };
    l.st = seg(rows * nch * sizeof(double2));
    l.part = seg((size_t)kSlots * rows * nch * sizeof(double));
    l.mz = seg(rows * sizeof(double2));
    l.rec = seg((size_t)kLevels * rows * sizeof(Rec));
    l.fin = seg(rows * sizeof(Fin));
    l.kc = seg(rows * sizeof(int2));
    l.dec = seg(rows * sizeof(int32_t));
    l.c0 = seg(rows * sizeof(Cand));
    l.cand = seg((size_t)total_nodes * sizeof(Cand));
    l.bad = seg((size_t)batch * sizeof(int32_t));
    l.total = (off + 255) & ~(size_t)255;
    return l;
}

struct SArgs {
    const int32_t *parent, *draft, *cu;
    int batch, total, rows, max_depth, vocab, nchunks;
    const void *root_logits, *node_logits;
    const float *root_q, *node_q;
    const double *u_accept, *u_final;
    double inv_t;
    ExpConst ek;
    double2 *st;    // [rows, nchunks] chunk (max, sum)
    double *part;   // [kSlots, rows, nchunks] residual chunk sums, slot s at s - 1
    double2 *mz;    // [rows] (M, Z), written for rows with candidates
    Rec *rec;       // [kLevels, rows], level L at L - 1
    Fin *fin;       // [rows]
    int2 *kc;       // [rows] (candidates tested, first index into cand)
    int32_t *dec;   // [rows] the accepted child, kDecFinal or kDecContinue
    Cand *c0;       // [rows] the row's first candidate
    Cand *cand;     // [T] candidates, each parent's in a run
    int32_t *bad;   // [B] 1: the request was answered by prep with an error
    int32_t *accept_len, *accept_idx, *next_token, *err;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

template <bool BF16>
__device__ __forceinline__ const char *logit_row(const SArgs &a, int row) {
    constexpr int64_t es = BF16 ? 2 : 4;
    return row < a.batch ? reinterpret_cast<const char *>(a.root_logits) + (int64_t)row * a.vocab * es
                         : reinterpret_cast<const char *>(a.node_logits) + (int64_t)(row - a.batch) * a.vocab * es;
}
__device__ __forceinline__ const float *q_row(const SArgs &a, int row) {
    return row < a.batch ? a.root_q + (int64_t)row * a.vocab : a.node_q + (int64_t)(row - a.batch) * a.vocab;
}
template <bool BF16>
__device__ __forceinline__ float logit_at(const char *rb, int i) {
    return BF16 ? bf16_lo(reinterpret_cast<const uint16_t *>(rb)[i]) : reinterpret_cast<const float *>(rb)[i];
}

// A lane's 32 logits of the chunk starting at c0: element 4g + h of the lane
// is index c0 + (64 g + lane) * 4 + h (g < 8, h < 4), so each load
// instruction of the wave reads one contiguous run.  Indices at or past
// vocab read -inf.  `vec`: rows start 16-byte aligned (vocab % 4 == 0).
template <bool BF16>
__device__ __forceinline__ void load_logits(const char *rb, int vocab, int c0, int lane, bool vec,
                                            float x[kPerLane]) {
    if (vec && c0 + kChunk <= vocab) {
        if (BF16) {
            const uint2 *p = reinterpret_cast<const uint2 *>(rb + (int64_t)c0 * 2);
            uint2 w[kPerLane / 4];
#pragma unroll
            for (int g = 0; g < kPerLane / 4; ++g) w[g] = p[g * 64 + lane];
#pragma unroll
            for (int g = 0; g < kPerLane / 4; ++g) {
                x[4 * g] = bf16_lo(w[g].x);
                x[4 * g + 1] = bf16_hi(w[g].x);
                x[4 * g + 2] = bf16_lo(w[g].y);
                x[4 * g + 3] = bf16_hi(w[g].y);
            }
        } else {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(rb + (int64_t)c0 * 4);
            u32x4 w[kPerLane / 4];
#pragma unroll
            for (int g = 0; g < kPerLane / 4; ++g) w[g] = p[g * 64 + lane];
#pragma unroll
            for (int g = 0; g < kPerLane / 4; ++g)
#pragma unroll
                for (int h = 0; h < 4; ++h) x[4 * g + h] = __uint_as_float(w[g][h]);
        }
        return;
    }
#pragma unroll
    for (int g = 0; g < kPerLane / 4; ++g)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int i = c0 + (g * 64 + lane) * 4 + h;
            x[4 * g + h] = i < vocab ? logit_at<BF16>(rb, i) : -INFINITY;
        }
}
// The draft probabilities at the same indices (0 past vocab).
__device__ __forceinline__ void load_q(const float *qr, int vocab, int c0, int lane, bool vec, float q[kPerLane]) {
    if (vec && c0 + kChunk <= vocab) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(qr + c0);
        u32x4 w[kPerLane / 4];
#pragma unroll
        for (int g = 0; g < kPerLane / 4; ++g) w[g] = p[g * 64 + lane];
#pragma unroll
        for (int g = 0; g < kPerLane / 4; ++g)
#pragma unroll
            for (int h = 0; h < 4; ++h) q[4 * g + h] = __uint_as_float(w[g][h]);
        return;
    }
#pragma unroll
    for (int g = 0; g < kPerLane / 4; ++g)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int i = c0 + (g * 64 + lane) * 4 + h;
            q[4 * g + h] = i < vocab ? qr[i] : 0.0f;
        }
}

// p(v) = exp(y - M) / Z, as a product with iZ = 1 / Z.
__device__ __forceinline__ double p_of(float x, double inv_t, double M, double iZ, const double *etab,
                                       const ExpConst &ek) {
    return exp_nonpos((double)x * inv_t - M, etab, ek) * iZ;
}
// The unnormalised residual weight (p - c q)+ of one element.
__device__ __forceinline__ double resid(double p, double c, float q) { return fmax(p - c * (double)q, 0.0); }

// The chunk's sum of (p - c q)+ over a lane's 32 elements, then the wave.
__device__ __forceinline__ double chunk_resid_sum(const float x[kPerLane], const float q[kPerLane], double c,
                                                  double inv_t, double M, double iZ, const double *etab,
                                                  const ExpConst &ek) {
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) s += resid(p_of(x[e], inv_t, M, iZ, etab, ek), c, q[e]);
    return wave_sum64(s);
}

// The row's M = max y and Z = sum exp(y - M) from its chunk statistics, by
// one wavefront: lane l takes chunks l, l + 64, ... in order, then a
// butterfly, so every wave of the row gets bit-identical values.  v0 and v1
// are chunks lane and lane + 64, loaded by the caller ((-inf, 0) past the
// row's chunks).
__device__ __forceinline__ double2 row_mz(const double2 *st, int nchunks, int lane, double2 v0, double2 v1,
                                          const double *etab, const ExpConst &ek) {
    double m = fmax(v0.x, v1.x);
    for (int c = lane + 128; c < nchunks; c += 64) m = fmax(m, st[c].x);
    m = wave_max64(m);
    double z = 0.0;
    if (v0.x > -INFINITY) z += v0.y * exp_nonpos(v0.x - m, etab, ek);
    if (v1.x > -INFINITY) z += v1.y * exp_nonpos(v1.x - m, etab, ek);
    for (int c = lane + 128; c < nchunks; c += 64) {
        const double2 v = st[c];
        if (v.x > -INFINITY) z += v.y * exp_nonpos(v.x - m, etab, ek);
    }
    return make_double2(m, wave_sum64(z));
}
// The sum of a row's residual chunk sums, the same way.
__device__ __forceinline__ double sum_chunks(const double *pc, int nchunks, int lane) {
    double s = 0.0;
    for (int c = lane; c < nchunks; c += 64) s += pc[c];
    return wave_sum64(s);
}

// The acceptance test of one candidate against the residual (p - c q)+ / W.
__device__ __forceinline__ bool accepts(const Cand &cd, double c, double W, double inv_t, double M, double iZ,
                                        const double *etab, const ExpConst &ek) {
    const double rx = resid(p_of(cd.y, inv_t, M, iZ, etab, ek), c, cd.q) / W;
    const double qx = (double)cd.q;
    const double ax = qx > 0.0 ? fmin(1.0, rx / qx) : (rx > 0.0 ? 1.0 : 0.0);
    return cd.u < ax;
}

__device__ __forceinline__ void put_fin(Fin *f, double c, double W, int lev) {
    Fin v;
    v.c = c;
    v.W = W;
    v.lev = lev;
    v.pad = 0;
    *f = v;
}

// Per request: checks, depths, candidate lists, and the defaults of rows
// without candidates.
template <bool BF16>
__device__ void prep_request(const SArgs &a, int b) {
    __shared__ __align__(16) int s_pl[TV_MAX_NODES];  // parent of a live node, INT_MIN for the others
    __shared__ int s_jump[TV_MAX_NODES];              // pointer doubling: an ancestor and the distance to it
    __shared__ int s_dist[TV_MAX_NODES];
    __shared__ int s_first[TV_MAX_NODES];             // first candidate of parent v, at v + 1
    __shared__ int s_wsum[kFrontWaves];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int32_t *idx_out = a.accept_idx + (int64_t)b * a.max_depth;
    for (int i = tid; i < a.max_depth; i += kFrontThreads) idx_out[i] = -1;

    int lo;
    const int n = request_nodes(a.cu, b, a.total, TV_MAX_NODES, &lo);
    if (n < 0) {
        if (tid == 0) {
            report(a.err, TV_DEVERR_BAD_REQUEST, b);
            a.accept_len[b] = 0;
            a.next_token[b] = -1;
            a.bad[b] = 1;
            a.kc[b] = make_int2(0, 0);
        }
        return;
    }
    int pa = -1, d = -1, badn = 0;
    if (tid < n) {
        pa = a.parent[lo + tid];
        d = a.draft[lo + tid];
        if (pa < -1 || pa >= tid) {
            report(a.err, TV_DEVERR_BAD_PARENT, lo + tid);
            badn = 1;
        }
        if (d >= a.vocab) {
            report(a.err, TV_DEVERR_BAD_TOKEN, lo + tid);
            badn = 1;
        }
    }
    if (__syncthreads_or(badn)) {
        // the passes skip the request's rows
        if (tid < n) a.kc[a.batch + lo + tid] = make_int2(0, 0);
        if (tid == 0) {
            a.accept_len[b] = 0;
            a.next_token[b] = -1;
            a.bad[b] = 1;
            a.kc[b] = make_int2(0, 0);
        }
        return;
    }
    const bool live = tid < n && d >= 0;
    // level(v), the number of nodes on the root -> v path, by pointer
    // doubling (until every chain reaches the root: at most ten rounds)
    int jump = tid < n ? pa : -1, dist = 1;
    s_pl[tid] = live ? pa : INT_MIN;
    if (tid < n) {
        s_jump[tid] = jump;
        s_dist[tid] = dist;
    }
    for (int r = 0; r < 10; ++r) {
        if (!__syncthreads_or(jump >= 0)) break;
        int nj = jump, nd = dist;
        if (jump >= 0) {
            nd = dist + s_dist[jump];
            nj = s_jump[jump];
        }
        __syncthreads();
        if (tid < n) {
            s_jump[tid] = nj;
            s_dist[tid] = nd;
        }
        jump = nj;
        dist = nd;
    }
    __syncthreads();
    // thread v + 1 counts the live children of v (entries past n are
    // INT_MIN, and no node has a parent >= n - 1); each live node counts its
    // live siblings of lower index.  Four parents per LDS read.
    const int v = tid - 1;
    int kids = 0, rank = 0;
    const int4 *pl4 = reinterpret_cast<const int4 *>(s_pl);
    for (int g = 0; g < (n + 3) >> 2; ++g) {  // uniform: broadcast reads
        const int4 p4 = pl4[g];
        const int j0 = g * 4;
        kids += (p4.x == v) + (p4.y == v) + (p4.z == v) + (p4.w == v);
        rank += (p4.x == pa && j0 < tid) + (p4.y == pa && j0 + 1 < tid) + (p4.z == pa && j0 + 2 < tid) +
                (p4.w == pa && j0 + 3 < tid);
    }
    // exclusive scan of the counts in parent order: each parent's first slot
    int incl = kids;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) s_wsum[wv] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < kFrontWaves; ++w) before += w < wv ? s_wsum[w] : 0;
    const int first = before + incl - kids;
    if (tid < n) s_first[tid] = first;
    __syncthreads();
    // rows of v = -1 .. n-2 by thread v + 1 (the root's also when n = 0),
    // and of the last node (which has no children) by thread 0.  v's
    // children are tested while fewer than max_depth nodes are accepted,
    // i.e. while level(v) < max_depth (the root's level is 0).  Rows without
    // candidates end the walk with r = p.
    for (int k2 = 0; k2 < 2; ++k2) {
        const int vv = k2 == 0 ? v : n - 1;
        if (k2 == 0 ? tid >= max(n, 1) : (tid != 0 || n == 0)) continue;
        const int lev_v = vv < 0 ? 0 : s_dist[vv];
        const int row = vv < 0 ? b : a.batch + lo + vv;
        const int kk = (k2 == 0 && lev_v < a.max_depth) ? kids : 0;
        a.kc[row] = make_int2(kk, lo + (k2 == 0 ? first : 0));
        if (kk == 0) {
            a.dec[row] = kDecFinal;
            put_fin(a.fin + row, 0.0, 1.0, 0);
        }
    }
    if (live) {
        const int prow = pa < 0 ? b : a.batch + lo + pa;
        Cand cd;
        cd.t = lo + tid;
        cd.x = d;
        cd.y = logit_at<BF16>(logit_row<BF16>(a, prow), d);
        cd.q = q_row(a, prow)[d];
        cd.u = a.u_accept[lo + tid];
        a.cand[lo + s_first[pa + 1] + rank] = cd;
        if (rank == 0) a.c0[prow] = cd;
    }
    if (tid == 0) a.bad[b] = 0;
}

// Chunk statistics of 16 chunks of one row, one per wavefront.
template <bool BF16>
__device__ void chunk_stats(const SArgs &a, int sb) {
    __shared__ double etab[kExpTable];
    const int groups = (a.nchunks + kFrontWaves - 1) / kFrontWaves;
    const int row = sb / groups;
    const int chunk = (sb - row * groups) * kFrontWaves + (int)(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    exp_table_fill(etab);
    __syncthreads();
    if (chunk >= a.nchunks) return;  // (wave-uniform; after the only barrier)
    const bool vec = (a.vocab & 3) == 0;
    float x[kPerLane];
    load_logits<BF16>(logit_row<BF16>(a, row), a.vocab, chunk * kChunk, lane, vec, x);
    // x -> x * (1/T) rounds monotonically, so the maximum of the products is
    // the product of the maximum
    float xm = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) xm = fmaxf(xm, x[e]);
    const double mc = wave_max64((double)xm * a.inv_t);
    double s = 0.0;
    if (mc > -INFINITY) {
#pragma unroll
        for (int e = 0; e < kPerLane; ++e) s += exp_nonpos((double)x[e] * a.inv_t - mc, etab, a.ek);
    }
    s = wave_sum64(s);
    if (lane == 0) a.st[(int64_t)row * a.nchunks + chunk] = make_double2(mc, s);
}

// Workgroups 0 .. B-1 prepare the requests; the rest take chunk statistics.
// The two write disjoint data.
template <bool BF16>
__global__ void __launch_bounds__(kFrontThreads) stoch_front_kernel(SArgs a) {
    if ((int)blockIdx.x < a.batch) prep_request<BF16>(a, (int)blockIdx.x);
    else chunk_stats<BF16>(a, (int)blockIdx.x - a.batch);
}

// Pass j: test j of every open row, then the chunk sums of the next residual.
template <bool BF16>
__global__ void __launch_bounds__(64 * kPassWaves) stoch_pass_kernel(SArgs a, int j) {
    __shared__ double etab[kExpTable];
    const int groups = (a.nchunks + kPassWaves - 1) / kPassWaves;
    const int row = (int)(blockIdx.x / groups);
    const int chunk = (int)(blockIdx.x - row * groups) * kPassWaves + (int)(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const bool writer = chunk == 0 && lane == 0;
    const int64_t slot_elems = (int64_t)a.rows * a.nchunks;
    const int64_t rc0 = (int64_t)row * a.nchunks;
    Rec *rec_out = a.rec + (int64_t)j * a.rows + row;  // level j + 1
    // everything the decision reads, loaded together
    const int2 kc = a.kc[row];
    double c = 0.0, W = 1.0;
    int lev = 0;
    bool open;
    Cand cd;
    double2 mz = make_double2(0.0, 1.0);
    double2 v0 = make_double2(-INFINITY, 0.0), v1 = v0;  // pass 0: chunk statistics lane, lane + 64
    if (j == 0) {
        cd = a.c0[row];
        if (lane < a.nchunks) v0 = a.st[rc0 + lane];
        if (lane + 64 < a.nchunks) v1 = a.st[rc0 + lane + 64];
        open = kc.x > 0;
    } else {
        const Rec R = a.rec[(int64_t)(j - 1) * a.rows + row];
        mz = a.mz[row];
        // the sum pass j-1 split over the chunks; 0 keeps the residual
        const double S = sum_chunks(a.part + (int64_t)(j - 1) * slot_elems + rc0, a.nchunks, lane);
        open = R.status == kOpen;
        cd = R.next;
        c = R.c;
        W = R.W;
        lev = R.lev;
        if (S > 0.0) {
            c = R.c1;
            W = S;
            lev = j;
        }
    }
    // a closed row's workgroup (its waves share the row) leaves before the
    // exp table and the barrier
    if (!open) {
        if (writer) rec_out->status = kClosed;
        return;
    }
    exp_table_fill(etab);
    __syncthreads();
    if (chunk >= a.nchunks) return;  // (wave-uniform; after the only barrier)
    if (j == 0) {
        mz = row_mz(a.st + rc0, a.nchunks, lane, v0, v1, etab, a.ek);
        if (writer) a.mz[row] = mz;
    }
    const double M = mz.x, iZ = 1.0 / mz.y;
    if (j >= kc.x) {  // every candidate rejected: the draw comes from this residual
        if (writer) {
            put_fin(a.fin + row, c, W, lev);
            a.dec[row] = kDecFinal;
            rec_out->status = kClosed;
        }
        return;
    }
    if (accepts(cd, c, W, a.inv_t, M, iZ, etab, a.ek)) {
        if (writer) {
            a.dec[row] = cd.t;
            rec_out->status = kClosed;
        }
        return;
    }
    // rejected: the chunk's sum of the next residual
    const bool vec = (a.vocab & 3) == 0;
    float x[kPerLane], q[kPerLane];
    load_logits<BF16>(logit_row<BF16>(a, row), a.vocab, chunk * kChunk, lane, vec, x);
    load_q(q_row(a, row), a.vocab, chunk * kChunk, lane, vec, q);
    Cand nx;
    nx.t = -1;
    nx.x = -1;
    nx.y = 0.0f;
    nx.q = 0.0f;
    nx.u = 1.0;
    if (writer) {
        const int ni = kc.y + j + 1;
        if (j + 1 < kc.x && ni >= 0 && ni < a.total) nx = a.cand[ni];
    }
    const double c1 = c + W;
    const double s = chunk_resid_sum(x, q, c1, a.inv_t, M, iZ, etab, a.ek);
    if (lane == 0) a.part[(int64_t)j * slot_elems + rc0 + chunk] = s;
    if (writer) {
        Rec o;
        o.status = kOpen;
        o.lev = lev;
        o.c = c;
        o.W = W;
        o.c1 = c1;
        o.next = nx;
        o.pad[0] = o.pad[1] = 0;
        *rec_out = o;
        if (j == kLevels - 1) a.dec[row] = kDecContinue;
    }
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
    for (int w = 0; w < kSelWaves; ++w) {
        const double t = lds[w];
        if (w < wv) before += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + v;
}

// The tests of row `row` past the passes, by the whole workgroup.  Returns
// the accepted child (global node), or -1 with the final residual in
// (*c, *W, *lev).
template <bool BF16>
__device__ int continue_row(const SArgs &a, int row, const double *etab, double *s_red, double *c_out,
                            double *W_out, int *lev_out) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const Rec R = a.rec[(int64_t)(kLevels - 1) * a.rows + row];
    const int2 kc = a.kc[row];
    const double2 mz = a.mz[row];
    const double M = mz.x, iZ = 1.0 / mz.y;
    const int64_t slot_elems = (int64_t)a.rows * a.nchunks;
    const int64_t rc0 = (int64_t)row * a.nchunks;
    const char *lrow = logit_row<BF16>(a, row);
    const float *qrow = q_row(a, row);
    const bool vec = (a.vocab & 3) == 0;
    double c = R.c, W = R.W, c1 = R.c1;
    int lev = R.lev, slot = kLevels;
    // the last pass's sum, added up as the passes add theirs
    double S = sum_chunks(a.part + (int64_t)(slot - 1) * slot_elems + rc0, a.nchunks, lane);
    bool pending = true, stuck = false;
    for (int j = kLevels;; ++j) {  // uniform: every thread decides alike
        if (pending) {
            if (S > 0.0) {
                c = c1;
                W = S;
                lev = slot;
            } else {
                stuck = true;  // r is kept, and so is every later residual
            }
            pending = false;
        }
        const int ci = kc.y + j;
        if (j >= kc.x || ci < 0 || ci >= a.total) {
            *c_out = c;
            *W_out = W;
            *lev_out = lev;
            return -1;
        }
        const Cand cd = j == kLevels ? R.next : a.cand[ci];
        if (accepts(cd, c, W, a.inv_t, M, iZ, etab, a.ek)) return cd.t;
        if (stuck) continue;
        c1 = c + W;
        slot = lev == kLevels + 1 ? kLevels + 2 : kLevels + 1;  // never the slot r lives in
        double *pc = a.part + (int64_t)(slot - 1) * slot_elems + rc0;
        double ws = 0.0;
        for (int ch = wv; ch < a.nchunks; ch += kSelWaves) {
            float x[kPerLane], q[kPerLane];
            load_logits<BF16>(lrow, a.vocab, ch * kChunk, lane, vec, x);
            load_q(qrow, a.vocab, ch * kChunk, lane, vec, q);
            const double s = chunk_resid_sum(x, q, c1, a.inv_t, M, iZ, etab, a.ek);
            if (lane == 0) pc[ch] = s;
            ws += s;
        }
        if (lane == 0) s_red[wv] = ws;
        __syncthreads();
        S = 0.0;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) S += s_red[w];
        __syncthreads();
        pending = true;
    }
}

// Per request: the walk along the decisions, then the draw.
template <bool BF16>
__global__ void __launch_bounds__(kSelThreads) stoch_select_kernel(SArgs a) {
    __shared__ int s_dec[TV_MAX_NODES + 1];
    __shared__ double etab[kExpTable];
    __shared__ double red_d[kSelWaves];
    __shared__ int red_i[2][kSelWaves];
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    exp_table_fill(etab);
    int lo;
    const int n = request_nodes(a.cu, b, a.total, TV_MAX_NODES, &lo);
    if (n < 0 || a.bad[b]) return;  // (uniform; prep answered the request)
    for (int i = tid; i <= n; i += kSelThreads) s_dec[i] = a.dec[i == 0 ? b : a.batch + lo + i - 1];
    __syncthreads();
    // the walk, by every thread alike; a decision names a later node of the
    // same request (anything else, possible only when request ranges
    // overlap, ends the walk with r = p)
    int32_t *idx_out = a.accept_idx + (int64_t)b * a.max_depth;
    int cur = -1, L = 0;
    bool have = false;  // the final residual is in (fc, fW, flev)
    double fc = 0.0, fW = 1.0;
    int flev = 0;
    for (;;) {
        const int dv = s_dec[cur + 1];
        if (dv == kDecContinue) {
            const int t = continue_row<BF16>(a, cur < 0 ? b : a.batch + lo + cur, etab, red_d, &fc, &fW, &flev);
            if (tid == 0) s_dec[cur + 1] = t >= 0 ? t : kDecFinal;
            __syncthreads();
            have = t < 0;
            continue;
        }
        if (dv < 0) break;  // kDecFinal
        const int li = dv - lo;
        if (li <= cur || li >= n || L >= a.max_depth) {
            have = true;
            fc = 0.0;
            fW = 1.0;
            flev = 0;
            break;
        }
        if (tid == 0) idx_out[L] = li;
        ++L;
        cur = li;
        have = false;
    }
    if (tid == 0) a.accept_len[b] = L;
    const int erow = cur < 0 ? b : a.batch + lo + cur;
    if (!have) {
        const Fin f = a.fin[erow];
        fc = f.c;
        fW = f.W;
        flev = f.lev;
    }
    const int lev = (flev >= 1 && flev <= kSlots) ? flev : 0;
    const int64_t rc0 = (int64_t)erow * a.nchunks;
    const double2 *st = a.st + rc0;
    const double *pc = a.part + (int64_t)(lev > 0 ? lev - 1 : 0) * a.rows * a.nchunks + rc0;
    // M from the chunk maxima (exact in any order); a residual's rows also
    // need the Z its passes used
    double M = -INFINITY;
    for (int ch = lane; ch < a.nchunks; ch += 64) M = fmax(M, st[ch].x);
    M = wave_max64(M);
    const double iZ = lev > 0 ? 1.0 / a.mz[erow].y : 1.0;
    // chunk weights: r = p weighs exp(y - M), so a chunk weighs
    // s_c exp(m_c - M); a residual's chunk weighs its chunk sum
    auto chunk_w = [&](int ch) -> double {
        if (ch >= a.nchunks) return 0.0;
        if (lev > 0) return pc[ch];
        const double2 v = st[ch];
        return v.x > -INFINITY ? v.y * exp_nonpos(v.x - M, etab, a.ek) : 0.0;
    };
    const int tiles = (a.nchunks + kSelThreads - 1) / kSelThreads;
    // 1. total weight and the last chunk with a positive weight
    const double w0 = chunk_w(tid);
    double tot0;
    const double incl0 = block_scan_d(w0, red_d, &tot0);
    double S = tot0;
    int last_pos = w0 > 0.0 ? tid : -1;
    for (int t = 1; t < tiles; ++t) {
        const int ch = t * kSelThreads + tid;
        const double w = chunk_w(ch);
        if (w > 0.0) last_pos = ch;
        double tot;
        block_scan_d(w, red_d, &tot);
        S += tot;
    }
    last_pos = wave_max_i(last_pos);
    if (lane == 0) red_i[1][wv] = last_pos;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) last_pos = max(last_pos, red_i[1][w]);
    __syncthreads();
    // 2. the first chunk whose running sum exceeds u * S
    const double target = a.u_final[b] * S;
    double base = 0.0;
    int found = INT_MAX;
    double found_base = 0.0;
    for (int t = 0; t < tiles && found == INT_MAX; ++t) {
        const int ch = t * kSelThreads + tid;
        double w, incl, tot;
        if (t == 0) {
            w = w0;
            incl = incl0;
            tot = tot0;
        } else {
            w = chunk_w(ch);
            incl = block_scan_d(w, red_d, &tot);
        }
        const int cand = (ch < a.nchunks && base + incl > target) ? ch : INT_MAX;
        const int wmin = wave_min_i(cand);
        if (lane == 0) red_i[0][wv] = wmin;
        if (cand != INT_MAX && cand == wmin) red_d[wv] = base + (incl - w);
        __syncthreads();
        int best = INT_MAX, bw = -1;
#pragma unroll
        for (int w2 = 0; w2 < kSelWaves; ++w2)
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
    // no crossing (u * S rounds to >= S): the last positive weight, by an
    // element scan that never crosses
    const bool fallback = found == INT_MAX;
    const int chunk = fallback ? max(last_pos, 0) : found;
    const double cbase = fallback ? 0.0 : found_base;
    const double ctarget = fallback ? INFINITY : target;
    // 3. the element: the chunk's weights in index order
    const char *lrow = logit_row<BF16>(a, erow);
    const float *qrow = q_row(a, erow);
    const int i0 = chunk * kChunk + tid * kSelPer;
    double w[kSelPer];
    double own = 0.0;
    int last_i = -1;
#pragma unroll
    for (int k = 0; k < kSelPer; ++k) {
        const int i = i0 + k;
        double wk = 0.0;
        if (i < a.vocab) {
            const float xk = logit_at<BF16>(lrow, i);
            if (lev > 0) {
                wk = resid(p_of(xk, a.inv_t, M, iZ, etab, a.ek), fc, qrow[i]);
            } else {
                const double y = (double)xk * a.inv_t;
                wk = y > -INFINITY ? exp_nonpos(y - M, etab, a.ek) : 0.0;
            }
        }
        w[k] = wk;
        own += wk;
        if (wk > 0.0) last_i = i;
    }
    double tot;
    const double incl = block_scan_d(own, red_d, &tot);
    double run = cbase + (incl - own);
    int cand = INT_MAX;
#pragma unroll
    for (int k = 0; k < kSelPer; ++k) {
        run += w[k];
        if (cand == INT_MAX && run > ctarget) cand = i0 + k;
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
        for (int w2 = 0; w2 < kSelWaves; ++w2) {
            first = min(first, red_i[0][w2]);
            last = max(last, red_i[1][w2]);
        }
        a.next_token[b] = first != INT_MAX ? first : (last >= 0 ? last : 0);
    }
}

template <bool BF16>
void launch_all(const SArgs &a, hipStream_t stream) {
    const int64_t front = (int64_t)a.batch + (int64_t)a.rows * ((a.nchunks + kFrontWaves - 1) / kFrontWaves);
    const int64_t pass = (int64_t)a.rows * ((a.nchunks + kPassWaves - 1) / kPassWaves);
    hipLaunchKernelGGL(stoch_front_kernel<BF16>, dim3((unsigned)front), dim3(kFrontThreads), 0, stream, a);
    for (int j = 0; j < kLevels; ++j)
        hipLaunchKernelGGL(stoch_pass_kernel<BF16>, dim3((unsigned)pass), dim3(64 * kPassWaves), 0, stream, a, j);
    hipLaunchKernelGGL(stoch_select_kernel<BF16>, dim3(a.batch), dim3(kSelThreads), 0, stream, a);
}

}  // namespace

size_t accept_stochastic_workspace(int batch, int total_nodes, int vocab) {
    return layout(batch, total_nodes, vocab).total;
}

hipError_t launch_accept_stochastic(const int32_t *parent, const int32_t *draft, const int32_t *cu_nodes, int batch,
                                    int total_nodes, int max_depth, const void *root_logits,
                                    const void *node_logits, tv_dtype dtype, double inv_t, const float *root_q,
                                    const float *node_q, int vocab, const double *u_accept, const double *u_final,
                                    int32_t *accept_len, int32_t *accept_idx, int32_t *next_token, void *workspace,
                                    int32_t *err, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    const Layout l = layout(batch, total_nodes, vocab);
    char *ws = reinterpret_cast<char *>(workspace);
    SArgs a;
    a.parent = parent;
    a.draft = draft;
    a.cu = cu_nodes;
    a.batch = batch;
    a.total = total_nodes;
    a.rows = batch + total_nodes;
    a.max_depth = max_depth;
    a.vocab = vocab;
    a.nchunks = (vocab + kChunk - 1) / kChunk;
    a.root_logits = root_logits;
    a.node_logits = node_logits;
    a.root_q = root_q;
    a.node_q = node_q;
    a.u_accept = u_accept;
    a.u_final = u_final;
    a.inv_t = inv_t;
    a.ek = exp_const();
    a.st = reinterpret_cast<double2 *>(ws + l.st);
    a.part = reinterpret_cast<double *>(ws + l.part);
    a.mz = reinterpret_cast<double2 *>(ws + l.mz);
    a.rec = reinterpret_cast<Rec *>(ws + l.rec);
    a.fin = reinterpret_cast<Fin *>(ws + l.fin);
    a.kc = reinterpret_cast<int2 *>(ws + l.kc);
    a.dec = reinterpret_cast<int32_t *>(ws + l.dec);
    a.c0 = reinterpret_cast<Cand *>(ws + l.c0);
    a.cand = reinterpret_cast<Cand *>(ws + l.cand);
    a.bad = reinterpret_cast<int32_t *>(ws + l.bad);
    a.accept_len = accept_len;
    a.accept_idx = accept_idx;
    a.next_token = next_token;
    a.err = err;
    if (dtype == TV_BF16) launch_all<true>(a, stream);
    else launch_all<false>(a, stream);
    return hipGetLastError();
}

}  // namespace tv
