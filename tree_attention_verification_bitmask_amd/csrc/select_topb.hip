// tree_select_topb: the draft tree chosen in one step from a frontier ledger.
//
// [DT]  = "DominoTree: Conditional Tree-Structured Drafting with Domino for
//         Speculative Decoding" (arXiv 2607.08642), section 3.3 and
//         Appendix B: the ledger's global top B, ordered parents first,
//         parent pointers remapped, short trees padded with dead leaves.
// [DAR] = "DARTree: Speculative Diffusion Decoding with Autoregressive Draft
//         Trees" (gist.science), "2. Deferred Best-First Pruning": the same
//         global top B with a non-positive depth bonus beta.
//
// One workgroup of 1024 threads per request; the request's keys live in LDS.
//   1. key(e) = score + beta * level in double (exact widening, exact
//      product, one rounding), mapped to an unsigned integer that orders
//      like the key; empty slots (non-finite keys) map to 0.
//   2. The n-th largest key (n = min(B, finite slots)) by an MSB-first
//      radix select, 8 bits per pass over the 64-bit keys; each pass is one
//      LDS histogram and one scan by a single wave.  The search stops once
//      the bin holding the n-th key is needed whole.
//   3. Slots above the threshold are chosen, plus the first `need` slots
//      equal to it in slot order (depth, then lane): a block-wide prefix
//      count over contiguous per-thread ranges.
//   4. The chosen slots (at most 1024) are ranked by (key descending, slot
//      ascending): a group of threads per chosen slot counts the chosen
//      slots that precede it -- the rank is its output position.
//   5. Parent pointers are remapped through a slot -> position table in
//      LDS; a parent that is out of range, not chosen, or ranked later is a
//      bad ledger (the node becomes a dead leaf).
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kPerThread = TV_MAX_LEDGER / kSelThreads;  // slots per thread (contiguous)
static_assert(TV_MAX_LEDGER % kSelThreads == 0, "ledger slots split evenly over the threads");
static_assert(TV_MAX_NODES <= kSelThreads, "one chosen slot per thread in the ranking");

// LDS position of slot e's key.  Thread t owns slots t*kPerThread ..
// t*kPerThread + kPerThread - 1 (contiguous, so prefix counts follow slot
// order); storing slot e at (e % kPerThread) * kSelThreads + e / kPerThread
// makes the reads of one wave consecutive (free of bank conflicts).
__device__ __forceinline__ int kidx(int e) { return (e % kPerThread) * kSelThreads + e / kPerThread; }

// Unsigned image of a double that orders like the double (0 < every image of
// a finite value; NaN never reaches it).
__device__ __forceinline__ uint64_t order_bits(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4, 8 within each row of 16 lanes, then the last lane of row 0 (and
// of row 2) is added to row 1 (row 3), then lane 31 to rows 2 and 3.  Lanes
// without a source add 0.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// Block-wide exclusive prefix sum of one int per thread; also returns the
// total.  Uses `wsum` (kSelWaves ints of LDS).
__device__ __forceinline__ int block_exclusive_scan(int v, int *wsum, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int x = wave_inclusive_scan(v);
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const int s = wsum[w];
        if (w < wave) base += s;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

__global__ void __launch_bounds__(kSelThreads) select_topb_kernel(
    const float *__restrict__ score, const int32_t *__restrict__ parent, const int32_t *__restrict__ token,
    int depth, int lanes, int budget, float beta, int32_t *__restrict__ tree_parent,
    int32_t *__restrict__ tree_token, int32_t *__restrict__ n_real, int32_t *__restrict__ err) {
    __shared__ uint64_t skey[TV_MAX_LEDGER];
    __shared__ int16_t pos_of[TV_MAX_LEDGER];  // slot -> output position, -1 if not chosen
    __shared__ uint64_t ckey[TV_MAX_NODES];    // chosen slots, in slot order
    __shared__ int16_t cslot[TV_MAX_NODES];
    __shared__ int16_t slot_at[TV_MAX_NODES];  // output position -> slot
    __shared__ int hist[256];
    __shared__ int wsum[kSelWaves];
    __shared__ uint64_t s_prefix;
    __shared__ int s_need, s_done;

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int E = depth * lanes;
    const int64_t base = (int64_t)b * E;

    // 1. keys, read with coalesced loads (slot e = i * kSelThreads + tid)
    // and stored at kidx(e).
    int nfin = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int e = i * kSelThreads + tid;
        uint64_t k = 0;
        if (e < E) {
            const int t = e / lanes;
            double x = (double)score[base + e] + (double)beta * (double)(t + 1);
            if (x == 0.0) x = 0.0;  // -0 and +0 are one key
            if (isfinite(x)) {
                k = order_bits(x);
                ++nfin;
            }
        }
        skey[kidx(e)] = k;
        pos_of[e] = -1;
    }
    int nfin_total;
    (void)block_exclusive_scan(nfin, wsum, &nfin_total);  // (its barriers publish skey)
    const int nsel = min(budget, nfin_total);
    // this thread's contiguous slots, kept in registers from here on
    uint64_t kreg[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) kreg[i] = skey[i * kSelThreads + tid];

    // 2. the nsel-th largest key: prefix fixed 8 bits per pass, MSB first
    if (tid == 0) {
        s_prefix = 0;
        s_need = nsel;
        s_done = 0;
    }
    __syncthreads();
    uint64_t mask = 0;
    if (nsel > 0) {
        for (int d = 7; d >= 0; --d) {
            if (tid < 256) hist[tid] = 0;
            __syncthreads();
            const uint64_t prefix = s_prefix;
            const int lane = tid & 63;
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) {
                const uint64_t k = kreg[i];
                const bool v = k != 0 && (k & mask) == prefix;
                const int dg = v ? (int)((k >> (8 * d)) & 0xFF) : -1;
                // Lanes sharing a digit add it with one atomic (the high
                // digits of clustered keys collide); the rest add one each.
                uint64_t pend = __ballot(v);
                for (int it = 0; it < 4 && pend; ++it) {
                    const int leader = __builtin_ctzll(pend);
                    const int ld = __builtin_amdgcn_readlane(dg, leader);
                    const uint64_t same = __ballot(dg == ld) & pend;
                    if (__popcll(same) < 8) break;
                    if (lane == leader) atomicAdd(&hist[ld], __popcll(same));
                    pend &= ~same;
                }
                if ((pend >> lane) & 1) atomicAdd(&hist[dg], 1);
            }
            __syncthreads();
            if (tid < 64) {
                // lane l holds digits 255-4l .. 252-4l (high digits first)
                int c[4], s4 = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    c[q] = hist[255 - 4 * tid - q];
                    s4 += c[q];
                }
                const int incl = wave_inclusive_scan(s4);
                const int need = s_need;
                int above = incl - s4;  // keys with a higher digit than this lane's first
                const bool mine = above < need && need <= incl;
                if (mine) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (above + c[q] >= need) {
                            s_prefix = prefix | ((uint64_t)(255 - 4 * tid - q) << (8 * d));
                            s_need = need - above;
                            // the whole bin is needed: its keys need no finer split
                            s_done = c[q] == need - above;
                            break;
                        }
                        above += c[q];
                    }
                }
            }
            __syncthreads();
            mask |= 0xFFull << (8 * d);
            if (s_done) break;
        }
    }
    // Threshold on the bytes fixed so far: keys whose fixed bytes exceed it
    // are chosen, and the first need_eq of those equal to it in slot order
    // (all of them when the search stopped early).
    const uint64_t thr = s_prefix;
    const int need_eq = s_need;

    // 3. chosen: keys above the threshold, and the first need_eq equal to it
    int n_eq = 0, n_gt = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const uint64_t k = kreg[i] & mask;
        n_eq += (nsel > 0 && kreg[i] != 0 && k == thr) ? 1 : 0;
        n_gt += (nsel > 0 && k > thr) ? 1 : 0;
    }
    int eq_total;
    int eq_rank = block_exclusive_scan(n_eq, wsum, &eq_total);
    int my_sel = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const uint64_t k = kreg[i] & mask;
        if (nsel > 0 && kreg[i] != 0 && k == thr) my_sel += (eq_rank++ < need_eq) ? 1 : 0;
    }
    my_sel += n_gt;
    int sel_total;
    int at = block_exclusive_scan(my_sel, wsum, &sel_total);
    eq_rank -= n_eq;  // back to this thread's first equal slot
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int e = tid * kPerThread + i;
        const uint64_t k = kreg[i] & mask;
        bool take = false;
        if (nsel > 0 && k > thr) take = true;
        if (nsel > 0 && kreg[i] != 0 && k == thr) take = (eq_rank++ < need_eq);
        if (take) {
            ckey[at] = kreg[i];
            cslot[at] = (int16_t)e;
            ++at;
        }
    }
    __syncthreads();

    // 4. rank of each chosen slot = its output position.  A group of tpe
    // threads (a power of two dividing 64, so a group lies in one wave)
    // shares one chosen slot; each counts a strided part of the slots that
    // precede it, and the group sums its counts.
    if (nsel > 0) {
        int np2 = 1;
        while (np2 < nsel) np2 <<= 1;
        const int tpe = min(64, kSelThreads / np2);
        const int i = tid / tpe, sub = tid % tpe;
        int r = 0, e = 0;
        if (i < nsel) {
            const uint64_t k = ckey[i];
            e = cslot[i];
            for (int j = sub; j < nsel; j += tpe) {
                const uint64_t kj = ckey[j];
                r += (kj > k || (kj == k && cslot[j] < e)) ? 1 : 0;
            }
        }
        for (int off = tpe >> 1; off >= 1; off >>= 1) r += __shfl_xor(r, off, 64);
        if (i < nsel && sub == 0) {
            pos_of[e] = (int16_t)r;
            slot_at[r] = (int16_t)e;
        }
    }
    __syncthreads();

    // 5. outputs, with parent pointers remapped
    for (int i = tid; i < budget; i += kSelThreads) {
        int32_t tp = -1, tt = -1;
        if (i < nsel) {
            const int e = slot_at[i];
            const int t = e / lanes, slot = e - t * lanes;
            const int p = parent[base + e];
            bool ok;
            if (t == 0) {
                ok = p == -1;
            } else {
                ok = p >= 0 && p < lanes;
                if (ok) {
                    const int pp = pos_of[(t - 1) * lanes + p];
                    ok = pp >= 0 && pp < i;
                    tp = pp;
                }
            }
            if (ok) {
                tt = token[base + t * lanes + slot];
            } else {
                tp = -1;
                report(err, TV_DEVERR_BAD_LEDGER, b);
            }
        }
        tree_parent[(int64_t)b * budget + i] = tp;
        tree_token[(int64_t)b * budget + i] = tt;
    }
    if (tid == 0) n_real[b] = nsel;
}

}  // namespace

hipError_t launch_select_topb(const float *score, const int32_t *parent, const int32_t *token, int batch,
                              int depth, int lanes, int budget, float beta, int32_t *tree_parent,
                              int32_t *tree_token, int32_t *n_real, int32_t *err, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    hipLaunchKernelGGL(select_topb_kernel, dim3(batch), dim3(kSelThreads), 0, stream, score, parent, token,
                       depth, lanes, budget, beta, tree_parent, tree_token, n_real, err);
    return hipGetLastError();
}

}  // namespace tv
