// Tree-aware recurrent verification for a Gated-DeltaNet layer.
//
// [DT] = "DominoTree: Conditional Tree-Structured Drafting with Domino for
// Speculative Decoding" (arXiv 2607.08642), section 4.5.4, "Tree-aware
// recurrent verification": an ancestor mask is not enough for a recurrent
// layer.  Every node needs the recurrent state of its own root path and a
// dense short-convolution window made of its own ancestors, and only the
// accepted path's state is committed.  A chain recurrence over the flattened
// tree would let a rejected sibling write into the state its cousins read.
//
// The page gives no formulas; the layer is the gated delta rule with L2-normalised
// queries and keys:
//   S_t = e^{g_t} S_p (I - beta_t k^_t k^_t^T) + beta_t v_t k^_t^T,  o_t = S_t q^_t
// where p = parent(t), the request's committed state S0 stands in for the
// parent of a root child, S is [dv, dk] per value head, and value head h reads
// query/key head h / (Hv / Hk).
//
// gdn_conv_kernel: the depthwise causal convolution (width K) with SiLU.  A
// node's window is the committed conv state followed by the inputs along its
// root path, i.e. its K nearest ancestors-or-self, topped up from the conv
// state.  Streaming work: one thread per (node, 8 channels).
//
// gdn_verify_kernel: all nodes' outputs in one pass per (request, value head,
// 32-channel slice of v).  The recurrence is unrolled with the
// ancestor-restricted WY form: writing S_t = e^{G_t} S0 + sum_{s in path(t)}
// e^{G_t - G_s} u_s k^_s^T (G = log decay summed along the root path), the
// write vectors satisfy
//   u_t + sum_{s in anc(t)} A[t,s] u_s = r_t,
//   A[t,s] = beta_t e^{G_t - G_s} (k^_t . k^_s),  r_t = beta_t (v_t - e^{G_t} S0 k^_t)
// and o_t = e^{G_t} S0 q^_t + sum_{s in path(t)} c[t,s] u_s with
// c[t,s] = e^{G_t - G_s} (q^_t . k^_s).  Both sums run over one root path only,
// so each node eliminates u on its own path: z^T (I + A_path) = c^T by back
// substitution, and o_t = e^{G_t} S0 q^_t + sum_a z_a r_{s_a}.  The dense
// products (K K^T, Q K^T, S0 K^T, S0 Q^T) run on v_mfma_f32_32x32x16_bf16; the
// fp32 state enters them as a bf16 hi + lo pair (about 16 significant bits,
// two products).  Only the entries on ancestor pairs are kept, in per-node
// tables indexed by the ancestor's level.
//
// gdn_commit_kernel: the accepted path's tokens replayed in order into the
// committed state (fp32, one step at a time), and the conv state advanced by
// the accepted inputs, in one launch.
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kHd = TV_GDN_HEAD_DIM;      // dk = dv
constexpr int kSlice = 32;                // value channels per verify workgroup
constexpr int kSlices = kHd / kSlice;
constexpr int kVThreads = 512;             // 8 waves: one 32-row block of nodes each
constexpr int kMaxN = TV_GDN_MAX_NODES;   // nodes per request
constexpr int kTab = TV_GDN_MAX_TABLE;    // nodes x max_depth per request
constexpr int kKRow = kHd + 8;            // LDS row of K in bf16 (272 B: rows 4 banks apart)
constexpr int kS0Row = kHd + 4;           // LDS row of the staged state slice in floats
constexpr float kEps = 1e-6f;
constexpr int kConvThreads = 256;

static_assert(kHd == 128, "fragments assume 128 channels per head");
static_assert(kMaxN * kKRow * 2 + kMaxN * kSlice * 4 + 2 * kTab * 4 + kTab * 2 + 6 * kMaxN * 4 + kMaxN * 2 <=
                  160 * 1024,
              "verify tables fit the 160 KB LDS");
static_assert(kMaxN * kSlice * 4 <= kMaxN * kKRow * 2, "S0 q per node fits over the K rows");
static_assert(kSlice * kS0Row <= 2 * kTab, "the staged state slice fits over the tables");

__device__ __forceinline__ float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// ---------------------------------------------------------------------------
// Convolution over each node's ancestor window.
// ---------------------------------------------------------------------------
template <int K>
__global__ void __launch_bounds__(kConvThreads) gdn_conv_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ cstate, const uint16_t *__restrict__ w,
    const int32_t *__restrict__ parent, const int32_t *__restrict__ cu_nodes, int batch, int C, int groups,
    uint16_t *__restrict__ y, int32_t *__restrict__ err) {
    const int t = blockIdx.x / groups;
    const int gi = blockIdx.x - t * groups;
    const bool reporter = gi == 0 && threadIdx.x == 0;
    const int b = request_of(cu_nodes, batch, t);
    if (b < 0) {
        if (reporter) report(err, TV_DEVERR_BAD_REQUEST, 0);
        return;
    }
    const int lo = cu_nodes[b];
    // a[j] = the node's j-th ancestor-or-self (local index), -1 past the root
    int a[K];
    int din = 0;
    int cur = t - lo;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        a[j] = cur;
        if (cur >= 0) {
            ++din;
            const int p = parent[lo + cur];
            const bool ok = p >= -1 && p < cur;
            if (!ok && reporter) report(err, TV_DEVERR_BAD_PARENT, lo + cur);
            cur = ok ? p : -1;
        }
    }
    const int c8 = (gi * kConvThreads + threadIdx.x) * 8;
    if (c8 >= C) return;
    // taps of the 8 channels: w[(c8 + e) * K + i], 8K contiguous bf16
    float wf[8][K];
    {
        const u32x4 *wp = reinterpret_cast<const u32x4 *>(w + (int64_t)c8 * K);
        uint32_t wv[4 * K];
#pragma unroll
        for (int i = 0; i < K; ++i) {
            const u32x4 q = wp[i];
            wv[4 * i] = q[0];
            wv[4 * i + 1] = q[1];
            wv[4 * i + 2] = q[2];
            wv[4 * i + 3] = q[3];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int i = 0; i < K; ++i) {
                const int f = e * K + i;
                wf[e][i] = (f & 1) ? bf16_hi(wv[f >> 1]) : bf16_lo(wv[f >> 1]);
            }
    }
    float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j) {
        // window slot K-1-j: the j-th ancestor-or-self, else conv state row
        // K-2-(j-din) (the most recent committed input is row K-2)
        const uint16_t *src = a[j] >= 0 ? x + (int64_t)(lo + a[j]) * C + c8
                                        : cstate + ((int64_t)b * (K - 1) + (K - 2 - (j - din))) * C + c8;
        const u32x4 q = *reinterpret_cast<const u32x4 *>(src);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xv = (e & 1) ? bf16_hi(q[e >> 1]) : bf16_lo(q[e >> 1]);
            z[e] = fmaf(wf[e][K - 1 - j], xv, z[e]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float y0 = z[2 * e] / (1.f + expf(-z[2 * e]));
        const float y1 = z[2 * e + 1] / (1.f + expf(-z[2 * e + 1]));
        o[e] = pack_bf16x2(y0, y1);
    }
    *reinterpret_cast<u32x4 *>(y + (int64_t)t * C + c8) = o;
}

// ---------------------------------------------------------------------------
// Verification: one workgroup per (request, value head, 32-channel slice).
// ---------------------------------------------------------------------------
struct VerifyArgs {
    const uint16_t *q, *k, *v;
    int64_t rs;  // row stride of q, k, v in elements
    const float *g, *beta, *state;
    const int32_t *parent, *cu_nodes;
    int batch, total_nodes, D, hk, hv;
    float scale;
    int l2norm;
    float *out;
    int32_t *err;
};

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t *p) { return *reinterpret_cast<const bf16x8_t *>(p); }

// Row of accumulator element e of lane l: 8 (e / 4) + 4 (l / 32) + e % 4 (its
// column is l % 32).
__device__ __forceinline__ int acc_row(int e, int half) { return 8 * (e >> 2) + 4 * half + (e & 3); }

__global__ void __launch_bounds__(kVThreads) gdn_verify_kernel(VerifyArgs p) {
    __shared__ __align__(16) uint16_t kS[kMaxN * kKRow];  // K rows (bf16); then S0 q per node (fp32 [t][32])
    __shared__ __align__(16) float rS[kMaxN * kSlice];     // v_t, then r_t, for the slice
    __shared__ __align__(16) float tabs[2 * kTab];         // S0 slice first; then Atab and Ctab
    float *const Atab = tabs;                              // [t][level-1]: k.k, then A[t, anc]
    float *const Ctab = tabs + kTab;                       // [t][level-1]: q.k, then c, then z
    __shared__ int16_t anc[kTab];                          // [t][level-1]: the ancestor at that level
    __shared__ __align__(16) float Gs[kMaxN], nk[kMaxN], mq[kMaxN], bt[kMaxN];
    __shared__ float gS[kMaxN];
    __shared__ int lev[kMaxN];
    __shared__ int16_t spar[kMaxN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // XCD-aware order: the 8 workgroups dealt to one XCD in a row are
    // consecutive tasks, so the tasks that read one key head share an L2.
    int id = blockIdx.x;
    const int nwg = gridDim.x;
    if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
    const int slice = id % kSlices;
    const int h = (id / kSlices) % p.hv;
    const int b = id / (kSlices * p.hv);
    const int D = p.D;
    int lo;
    const int n = request_nodes(p.cu_nodes, b, p.total_nodes, p.total_nodes, &lo);
    if (n < 0) {
        if (tid == 0) report(p.err, TV_DEVERR_BAD_REQUEST, b);
        return;
    }
    if (n > kMaxN || n * D > kTab) {
        if (tid == 0) report(p.err, TV_DEVERR_LIMIT, b);
        return;
    }
    if (n == 0) return;
    const int hkk = h / (p.hv / p.hk);
    const int i0 = slice * kSlice;
    const int nb = (n + 31) >> 5;
    const bool reporter = h == 0 && slice == 0;
    // Fragment of lane l: row l % 32, channels 16 ks + 8 (l / 32) .. + 8.
    // Wave w owns row block tb; waves w and w + 4 share a SIMD and get blocks
    // w and 7 - w, so the triangle's matrix work is balanced over the SIMDs.
    const int col = lane & 31, half = lane >> 5;
    const int tb = wave < 4 ? wave : 11 - wave;
    const bool has_tb = tb < nb;

    // ---- (0) every global load up front ---------------------------------------
    u32x4 kreg[kMaxN * 16 / kVThreads];
#pragma unroll
    for (int i = 0; i < kMaxN * 16 / kVThreads; ++i) {
        const int e = tid + i * kVThreads, row = e >> 4, g16 = e & 15;
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        if (row < n) kreg[i] = *reinterpret_cast<const u32x4 *>(p.k + (int64_t)(lo + row) * p.rs + hkk * kHd + 8 * g16);
    }
    int par_v = -1;
    float g_v = 0.f, b_v = 0.f;
    if (tid < n) {
        par_v = p.parent[lo + tid];
        g_v = p.g[(int64_t)(lo + tid) * p.hv + h];
        b_v = p.beta[(int64_t)(lo + tid) * p.hv + h];
    }
    bf16x8_t qa[8];
    {
        const int r = tb * 32 + col;
        const uint16_t *qrow = p.q + (int64_t)(lo + min(r, n - 1)) * p.rs + hkk * kHd + 8 * half;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            qa[ks] = bf16x8_t{};
            if (has_tb && r < n) qa[ks] = *reinterpret_cast<const bf16x8_t *>(qrow + 16 * ks);
        }
    }
    // v of the slice, row by row (4 threads per row, 8 channels each)
    u32x4 vreg[kMaxN * 4 / kVThreads];
#pragma unroll
    for (int i = 0; i < kMaxN * 4 / kVThreads; ++i) {
        const int e = tid + i * kVThreads, row = e >> 2;
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
        if (row < n)
            vreg[i] = *reinterpret_cast<const u32x4 *>(p.v + (int64_t)(lo + row) * p.rs + h * kHd + i0 + 8 * (e & 3));
    }
    // the state slice S0[i0 .. i0+31][:], coalesced (row = 32 threads x 4 floats)
    f32x4 sreg[kSlice * kHd / 4 / kVThreads];
    {
        const float *sbase = p.state + (((int64_t)b * p.hv + h) * kHd + i0) * kHd;
#pragma unroll
        for (int i = 0; i < kSlice * kHd / 4 / kVThreads; ++i)
            sreg[i] = *reinterpret_cast<const f32x4 *>(sbase + 4 * (tid + i * kVThreads));
    }
#pragma unroll
    for (int i = 0; i < kMaxN * 16 / kVThreads; ++i) {
        const int e = tid + i * kVThreads, row = e >> 4, g16 = e & 15;
        if (row < nb * 32) *reinterpret_cast<u32x4 *>(&kS[row * kKRow + 8 * g16]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < kMaxN * 4 / kVThreads; ++i) {
        const int e = tid + i * kVThreads, row = e >> 2;
        if (row < n) {
            float *dst = &rS[row * kSlice + 8 * (e & 3)];
            *reinterpret_cast<f32x4 *>(dst) =
                f32x4{bf16_lo(vreg[i][0]), bf16_hi(vreg[i][0]), bf16_lo(vreg[i][1]), bf16_hi(vreg[i][1])};
            *reinterpret_cast<f32x4 *>(dst + 4) =
                f32x4{bf16_lo(vreg[i][2]), bf16_hi(vreg[i][2]), bf16_lo(vreg[i][3]), bf16_hi(vreg[i][3])};
        }
    }
#pragma unroll
    for (int i = 0; i < kSlice * kHd / 4 / kVThreads; ++i) {
        const int e = 4 * (tid + i * kVThreads);
        *reinterpret_cast<f32x4 *>(&tabs[(e / kHd) * kS0Row + e % kHd]) = sreg[i];
    }
    if (tid < n) {
        spar[tid] = (int16_t)max(-2, min(par_v, kMaxN));
        gS[tid] = g_v;
        bt[tid] = b_v;
    }
    __syncthreads();

    // ---- (1) levels, ancestor rows, cumulative log decay (in LDS); norms --------
    if (tid < n) {
        const int t = tid;
        int16_t *row = &anc[t * D];
        int L = 0, u = t;
        float G = 0.f;
        // node first, then reversed in place (root first)
        while (u >= 0) {
            if (L == D) {
                if (reporter) report(p.err, TV_DEVERR_TOO_DEEP, lo + t);
                break;
            }
            row[L++] = (int16_t)u;
            G += gS[u];
            const int pp = spar[u];
            if (pp < -1 || pp >= u) {
                if (reporter) report(p.err, TV_DEVERR_BAD_PARENT, lo + u);
                break;
            }
            u = pp;
        }
        for (int j = 0; j < L / 2; ++j) {
            const int16_t x0 = row[j], x1 = row[L - 1 - j];
            row[j] = x1;
            row[L - 1 - j] = x0;
        }
        lev[t] = L;
        Gs[t] = G;
    }
    // S0 as the B operand of S0 k and S0 q: B[kk][j] = S0[i0 + j][kk], as hi + lo
    bf16x8_t sh[8], sl[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const float *src = &tabs[col * kS0Row + 16 * ks + 8 * half];
        const f32x4 s0 = *reinterpret_cast<const f32x4 *>(src);
        const f32x4 s1 = *reinterpret_cast<const f32x4 *>(src + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xv = e < 4 ? s0[e] : s1[e - 4];
            const __bf16 hb = (__bf16)xv;
            sh[ks][e] = hb;
            sl[ks][e] = (__bf16)(xv - (float)hb);
        }
    }
    if (has_tb) {
        const int r = tb * 32 + col;
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8_t kf = lds_frag(&kS[r * kKRow + 16 * ks + 8 * half]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float kx = (float)kf[e], qx = (float)qa[ks][e];
                sk = fmaf(kx, kx, sk);
                sq = fmaf(qx, qx, sq);
            }
        }
        sk += __shfl_xor(sk, 32, 64);
        sq += __shfl_xor(sq, 32, 64);
        if (half == 0 && r < n) {
            nk[r] = p.l2norm ? 1.f / sqrtf(sk + kEps) : 1.f;
            mq[r] = p.scale * (p.l2norm ? 1.f / sqrtf(sq + kEps) : 1.f);
        }
    }
    __syncthreads();

    // ---- (2) dense products on the matrix cores ------------------------------
    const f32x16_t zero16 = {};
    f32x16_t qs_acc = zero16;
    if (has_tb) {
        bf16x8_t ka[8];
        const int r = tb * 32 + col;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) ka[ks] = lds_frag(&kS[r * kKRow + 16 * ks + 8 * half]);
        f32x16_t ks_acc = zero16, qsa = zero16;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            ks_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], sh[ks], ks_acc, 0, 0, 0);
            qsa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks], sh[ks], qsa, 0, 0, 0);
            ks_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], sl[ks], ks_acc, 0, 0, 0);
            qsa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks], sl[ks], qsa, 0, 0, 0);
        }
        qs_acc = qsa;
        // the 16 rows of the lane's accumulator: 4 groups of 4 consecutive nodes
        int levt[16];
        {
            float gt[16], nt[16], btt[16], vt[16];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int t0 = tb * 32 + 8 * g4 + 4 * half;
                const f32x4 G4 = *reinterpret_cast<const f32x4 *>(&Gs[t0]);
                const f32x4 n4 = *reinterpret_cast<const f32x4 *>(&nk[t0]);
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&bt[t0]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    gt[4 * g4 + j] = G4[j];
                    nt[4 * g4 + j] = n4[j];
                    btt[4 * g4 + j] = b4[j];
                    levt[4 * g4 + j] = lev[t0 + j];
                }
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) vt[e] = rS[(tb * 32 + acc_row(e, half)) * kSlice + col];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = tb * 32 + acc_row(e, half);
                if (t < n) rS[t * kSlice + col] = btt[e] * (vt[e] - __expf(gt[e]) * nt[e] * ks_acc[e]);
                else levt[e] = 0;
            }
        }
        // k.k and q.k against every earlier row block; keep ancestor pairs
        for (int sb = 0; sb <= tb; ++sb) {
            bf16x8_t kb[8];
            const int sr = sb * 32 + col;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) kb[ks] = lds_frag(&kS[sr * kKRow + 16 * ks + 8 * half]);
            f32x16_t kk = zero16, qk = zero16;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                kk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], kb[ks], kk, 0, 0, 0);
                qk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks], kb[ks], qk, 0, 0, 0);
            }
            // the lane's column is node sr; element e's row is node t
            const int ls = sr < n ? lev[sr] : kMaxN;
            int at[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = tb * 32 + acc_row(e, half);
                at[e] = anc[min(t * D + ls - 1, kTab - 1)];
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = tb * 32 + acc_row(e, half);
                if (ls <= levt[e] && at[e] == sr) {
                    Atab[t * D + ls - 1] = kk[e];
                    Ctab[t * D + ls - 1] = qk[e];
                }
            }
        }
    }
    __syncthreads();

    // ---- (3) S0 q to LDS over the dead K rows; each node scales its rows -------
    float *qsS = reinterpret_cast<float *>(kS);
    if (has_tb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int t = tb * 32 + acc_row(e, half);
            if (t < n) qsS[t * kSlice + col] = qs_acc[e];
        }
    }
    if (tid < n) {
        const int t = tid;
        const int L = lev[t];
        const float Gt = Gs[t], bn = bt[t] * nk[t], mt = mq[t];
        float *arow = &Atab[t * D];
        float *crow = &Ctab[t * D];
        if (L <= 16) {
            // loads first (independent), then the products
            int sa[16];
            float gs[16], ns[16], av[16], cv[16];
#pragma unroll
            for (int a = 0; a < 16; ++a)
                if (a < L) {
                    sa[a] = anc[t * D + a];
                    av[a] = arow[a];
                    cv[a] = crow[a];
                }
#pragma unroll
            for (int a = 0; a < 16; ++a)
                if (a < L) {
                    gs[a] = Gs[sa[a]];
                    ns[a] = nk[sa[a]];
                }
#pragma unroll
            for (int a = 0; a < 16; ++a)
                if (a < L) {
                    const float f = __expf(Gt - gs[a]) * ns[a];
                    arow[a] = av[a] * bn * f;
                    crow[a] = cv[a] * mt * f;
                }
        } else {
            for (int a = 0; a < L; ++a) {
                const int s_ = anc[t * D + a];
                const float f = __expf(Gt - Gs[s_]) * nk[s_];
                arow[a] *= bn * f;
                crow[a] *= mt * f;
            }
        }
    }
    __syncthreads();

    // ---- (4) per node: z^T (I + A_path) = c^T by back substitution ------------
    // z_a is final once every deeper a' has been eliminated.
    if (tid < n) {
        const int t = tid;
        const int L = lev[t];
        float *crow = &Ctab[t * D];
        if (L <= 16) {
            float c[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                c[j] = 0.f;
                if (j < L) c[j] = crow[j];
            }
#pragma unroll
            for (int a = 15; a >= 1; --a) {
                if (a < L) {
                    const float za = c[a];
                    const float *arow = &Atab[anc[t * D + a] * D];
#pragma unroll
                    for (int j = 0; j < a; ++j) c[j] = fmaf(-za, arow[j], c[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (j < L) crow[j] = c[j];
        } else {
            for (int a = L - 1; a >= 1; --a) {
                const float za = crow[a];
                const float *arow = &Atab[anc[t * D + a] * D];
                for (int j = 0; j < a; ++j) crow[j] = fmaf(-za, arow[j], crow[j]);
            }
        }
    }
    __syncthreads();

    // ---- (5) outputs: thread = (node, 8 channels) --------------------------------
    {
        const int c0 = (tid & 3) * 8;
        for (int t = tid >> 2; t < n; t += kVThreads / 4) {
            const int L = lev[t];
            const float f = mq[t] * __expf(Gs[t]);
            f32x4 o0 = *reinterpret_cast<const f32x4 *>(&qsS[t * kSlice + c0]) * f;
            f32x4 o1 = *reinterpret_cast<const f32x4 *>(&qsS[t * kSlice + c0 + 4]) * f;
            const float *zr = &Ctab[t * D];
            const int16_t *ar = &anc[t * D];
#pragma unroll 4
            for (int a = 0; a < L; ++a) {
                const float z = zr[a];
                const float *rr = &rS[ar[a] * kSlice + c0];
                const f32x4 r0 = *reinterpret_cast<const f32x4 *>(rr);
                const f32x4 r1 = *reinterpret_cast<const f32x4 *>(rr + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o0[e] = fmaf(z, r0[e], o0[e]);
                    o1[e] = fmaf(z, r1[e], o1[e]);
                }
            }
            float *op = p.out + ((int64_t)(lo + t) * p.hv + h) * kHd + i0 + c0;
            *reinterpret_cast<f32x4 *>(op) = o0;
            *reinterpret_cast<f32x4 *>(op + 4) = o1;
        }
    }
}

// ---------------------------------------------------------------------------
// Commit: the accepted tokens replayed into the state, and the conv state.
// ---------------------------------------------------------------------------
constexpr int kCThreads = 256;

// Checks request b's accepted path; returns L (>= 0) or -1 after reporting.
__device__ __forceinline__ int commit_path(const int32_t *cu_nodes, const int32_t *accept_len,
                                           const int32_t *accept_idx, int b, int total_nodes, int D,
                                           bool reporter, int32_t *err, int *lo_out, int32_t *s_idx) {
    int lo;
    const int n = request_nodes(cu_nodes, b, total_nodes, total_nodes, &lo);
    *lo_out = lo;
    const int L = accept_len[b];  // (read with the offsets; b < batch)
    if ((n < 0) | (L < 0) | (L > D) | (L > n)) {
        if (reporter && threadIdx.x == 0) report(err, TV_DEVERR_BAD_REQUEST, b);
        return -1;
    }
    bool bad = false;
    if ((int)threadIdx.x < L) {
        const int my = accept_idx[(int64_t)b * D + threadIdx.x];
        bad = my < 0 || my >= n;
        s_idx[threadIdx.x] = my;
    }
    if (__syncthreads_or(bad)) {
        if (reporter && threadIdx.x == 0) report(err, TV_DEVERR_BAD_PATH, b);
        return -1;
    }
    return L;
}

struct CommitArgs {
    float *state;
    uint16_t *cstate;
    const uint16_t *x, *k, *v;
    int64_t rs;
    const float *g, *beta;
    const int32_t *cu_nodes, *accept_len, *accept_idx;
    int total_nodes, D, hk, hv, l2norm, C, groups, state_wgs;
    int32_t *err;
};

// State: one workgroup per (request, value head, 32 state rows); thread =
// (row, 16 columns), S k reduced over the row's 8 threads.
constexpr int kCRows = 32;

__device__ __forceinline__ void commit_state(const CommitArgs &p, int wg) {
    __shared__ __align__(16) float khat[TV_MAX_DEPTH][kHd];
    __shared__ float vS[TV_MAX_DEPTH][kCRows];
    __shared__ float al[TV_MAX_DEPTH], be[TV_MAX_DEPTH];
    __shared__ int32_t s_idx[TV_MAX_DEPTH];
    constexpr int kBlocks = kHd / kCRows;
    const int rb = wg % kBlocks;
    const int bh = wg / kBlocks;
    const int b = bh / p.hv, h = bh - (bh / p.hv) * p.hv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the thread's state slice, loaded while the path is checked
    const int r = tid >> 3, c0 = (tid & 7) * 16;
    float *srow = p.state + (((int64_t)b * p.hv + h) * kHd + rb * kCRows + r) * kHd + c0;
    float s[16];
#pragma unroll
    for (int c = 0; c < 16; c += 4) {
        const f32x4 x4 = *reinterpret_cast<const f32x4 *>(srow + c);
        s[c] = x4[0];
        s[c + 1] = x4[1];
        s[c + 2] = x4[2];
        s[c + 3] = x4[3];
    }
    int lo;
    const int L = commit_path(p.cu_nodes, p.accept_len, p.accept_idx, b, p.total_nodes, p.D, h == 0 && rb == 0,
                              p.err, &lo, s_idx);
    if (L <= 0) return;
    const int hkk = h / (p.hv / p.hk);
    // normalised keys, the rows' values, decays and write strengths
    for (int j = wave; j < L; j += kCThreads / 64) {
        const int64_t t = lo + s_idx[j];
        const uint32_t pr = *reinterpret_cast<const uint32_t *>(p.k + t * p.rs + hkk * kHd + 2 * lane);
        const float vx = lane < kCRows ? bf(p.v[t * p.rs + h * kHd + rb * kCRows + lane]) : 0.f;
        const float k0 = bf16_lo(pr), k1 = bf16_hi(pr);
        const float ss = wave_sum(fmaf(k0, k0, k1 * k1));
        const float nf = p.l2norm ? 1.f / sqrtf(ss + kEps) : 1.f;
        khat[j][2 * lane] = k0 * nf;
        khat[j][2 * lane + 1] = k1 * nf;
        if (lane < kCRows) vS[j][lane] = vx;
        if (lane == 0) {
            al[j] = expf(p.g[t * p.hv + h]);
            be[j] = p.beta[t * p.hv + h];
        }
    }
    __syncthreads();
    for (int j = 0; j < L; ++j) {
        const float *kh = &khat[j][c0];
        float y = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) y = fmaf(s[c], kh[c], y);
        y += __shfl_xor(y, 1, 64);
        y += __shfl_xor(y, 2, 64);
        y += __shfl_xor(y, 4, 64);
        const float a = al[j];
        const float wgt = be[j] * (vS[j][r] - a * y);
#pragma unroll
        for (int c = 0; c < 16; ++c) s[c] = fmaf(wgt, kh[c], a * s[c]);
    }
#pragma unroll
    for (int c = 0; c < 16; c += 4) *reinterpret_cast<f32x4 *>(srow + c) = f32x4{s[c], s[c + 1], s[c + 2], s[c + 3]};
}

// Conv state: one workgroup per (request, 2048 channels); thread = 8 channels.
template <int K>
__device__ __forceinline__ void commit_conv(const CommitArgs &p, int wg) {
    __shared__ int32_t s_idx[TV_MAX_DEPTH];
    const int b = wg / p.groups;
    const int gi = wg - b * p.groups;
    int lo;
    const int L = commit_path(p.cu_nodes, p.accept_len, p.accept_idx, b, p.total_nodes, p.D, gi == 0, p.err, &lo,
                              s_idx);
    if (L <= 0) return;
    const int c8 = (gi * kCThreads + threadIdx.x) * 8;
    if (c8 >= p.C) return;
    // sequence = old rows 0 .. K-2, then the accepted inputs; keep the last K-1
    uint16_t *base = p.cstate + (int64_t)b * (K - 1) * p.C + c8;
    u32x4 nv[K - 1];
#pragma unroll
    for (int r = 0; r < K - 1; ++r) {
        const int q = L + r;
        const uint16_t *src =
            q < K - 1 ? base + (int64_t)q * p.C : p.x + (int64_t)(lo + s_idx[q - (K - 1)]) * p.C + c8;
        nv[r] = *reinterpret_cast<const u32x4 *>(src);
    }
#pragma unroll
    for (int r = 0; r < K - 1; ++r) *reinterpret_cast<u32x4 *>(base + (int64_t)r * p.C) = nv[r];
}

// One launch for both: the first state_wgs workgroups advance the recurrent
// state, the rest the conv state.
template <int K>
__global__ void __launch_bounds__(kCThreads) gdn_commit_kernel(CommitArgs p) {
    const int wg = blockIdx.x;
    if (wg < p.state_wgs) commit_state(p, wg);
    else commit_conv<K>(p, wg - p.state_wgs);
}

}  // namespace

hipError_t launch_gdn_conv(const void *x, const void *conv_state, const void *weight, const int32_t *parent,
                           const int32_t *cu_nodes, int batch, int total_nodes, int channels, int conv_k, void *y,
                           int32_t *err, hipStream_t stream) {
    if (batch == 0 || total_nodes == 0) return hipSuccess;
    const int groups = (channels / 8 + kConvThreads - 1) / kConvThreads;
    const dim3 grid((unsigned)((int64_t)total_nodes * groups));
    const auto *xp = (const uint16_t *)x;
    const auto *cp = (const uint16_t *)conv_state;
    const auto *wp = (const uint16_t *)weight;
    auto *yp = (uint16_t *)y;
    switch (conv_k) {
        case 2:
            hipLaunchKernelGGL(gdn_conv_kernel<2>, grid, dim3(kConvThreads), 0, stream, xp, cp, wp, parent, cu_nodes,
                               batch, channels, groups, yp, err);
            break;
        case 3:
            hipLaunchKernelGGL(gdn_conv_kernel<3>, grid, dim3(kConvThreads), 0, stream, xp, cp, wp, parent, cu_nodes,
                               batch, channels, groups, yp, err);
            break;
        default:
            hipLaunchKernelGGL(gdn_conv_kernel<4>, grid, dim3(kConvThreads), 0, stream, xp, cp, wp, parent, cu_nodes,
                               batch, channels, groups, yp, err);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_gdn_verify(const void *q, const void *k, const void *v, int64_t row_stride, const float *g,
                             const float *beta, const float *state, const int32_t *parent, const int32_t *cu_nodes,
                             int batch, int total_nodes, int max_depth, int hk, int hv, float scale, int l2norm,
                             float *out, int32_t *err, hipStream_t stream) {
    if (batch == 0 || total_nodes == 0) return hipSuccess;
    VerifyArgs a{(const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, row_stride, g, beta, state,
                 parent, cu_nodes, batch, total_nodes, max_depth, hk, hv, scale, l2norm, out, err};
    const int64_t grid = (int64_t)batch * hv * kSlices;
    hipLaunchKernelGGL(gdn_verify_kernel, dim3((unsigned)grid), dim3(kVThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_gdn_commit(float *state, void *conv_state, const void *x, const void *k, const void *v,
                             int64_t row_stride, const float *g, const float *beta, const int32_t *cu_nodes,
                             const int32_t *accept_len, const int32_t *accept_idx, int batch, int total_nodes,
                             int max_depth, int hk, int hv, int channels, int conv_k, int l2norm, int32_t *err,
                             hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    const int groups = (channels / 8 + kCThreads - 1) / kCThreads;
    const int state_wgs = batch * hv * (kHd / kCRows);
    CommitArgs a{state, (uint16_t *)conv_state, (const uint16_t *)x, (const uint16_t *)k, (const uint16_t *)v,
                 row_stride, g, beta, cu_nodes, accept_len, accept_idx, total_nodes, max_depth, hk, hv, l2norm,
                 channels, groups, state_wgs, err};
    const dim3 grid((unsigned)((int64_t)state_wgs + (int64_t)batch * groups));
    switch (conv_k) {
        case 2:
            hipLaunchKernelGGL(gdn_commit_kernel<2>, grid, dim3(kCThreads), 0, stream, a);
            break;
        case 3:
            hipLaunchKernelGGL(gdn_commit_kernel<3>, grid, dim3(kCThreads), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL(gdn_commit_kernel<4>, grid, dim3(kCThreads), 0, stream, a);
            break;
    }
    return hipGetLastError();
}

}  // namespace tv
