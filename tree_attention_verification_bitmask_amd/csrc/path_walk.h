// Device pieces shared by the acceptance walk and the path compaction, so the
// separate calls and the fused one run the same code.
//
// [TSD] = "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
// Tree Attention Accelerate LLM Serving" (llms.blog), sections "Verification
// and Acceptance Algorithms" (greedy tree verification) and "KV Cache
// Rollback".
#pragma once
#include "tv_device.h"

namespace tv {

constexpr int kWalkPerLane = (TV_MAX_NODES + 63) / 64;  // nodes held per lane

// The walk for a request too large to hold in registers: each step tests the
// candidates (parent == current, draft == wanted token) 64 at a time from
// global memory and a ballot picks the lowest matching index.  One wavefront;
// idx may point to global memory or LDS.
__device__ inline void walk_global(const int32_t *par, const int32_t *dr, const int32_t *tg, int n,
                                   int want, int max_depth, int32_t *idx, int32_t *len_out,
                                   int32_t *next_out) {
    const int lane = threadIdx.x & 63;
    int cur = -1;
    int len = 0;
    while (len < max_depth) {
        int found = -1;
        for (int base = 0; base < n; base += 64) {
            const int j = base + lane;
            bool m = false;
            if (j < n) {
                const int dj = dr[j];
                m = (par[j] == cur) && (dj >= 0) && (dj == want);
            }
            const unsigned long long bal = __ballot(m);
            if (bal) {
                found = base + __builtin_ctzll(bal);
                break;
            }
        }
        if (found < 0) break;
        if (lane == 0) idx[len] = found;
        ++len;
        cur = found;
        want = tg[found];
    }
    for (int j = len + lane; j < max_depth; j += 64) idx[j] = -1;
    if (lane == 0) {
        *len_out = len;
        *next_out = want;
    }
}

// Loads a request's parent, draft and target rows (n <= TV_MAX_NODES) into
// lane-held registers: lane l holds nodes l, l + 64, ...  Every load is
// issued before the target rows are stored to stg (LDS), so the wave pays one
// memory round trip, not one per 64 nodes.  The caller synchronises before
// walk_registers reads stg.
__device__ inline void walk_load(const int32_t *par, const int32_t *dr, const int32_t *tg, int n,
                                 int (&pk)[kWalkPerLane], int (&dk)[kWalkPerLane], int32_t *stg) {
    const int lane = threadIdx.x & 63;
    const int nk = (n + 63) / 64;
    int tk[kWalkPerLane];
#pragma unroll
    for (int k = 0; k < kWalkPerLane; ++k) {
        const int j = 64 * k + lane;
        pk[k] = -2;
        dk[k] = -1;
        tk[k] = 0;
        if (k < nk && j < n) {
            pk[k] = par[j];
            dk[k] = dr[j];
            tk[k] = tg[j];
        }
    }
#pragma unroll
    for (int k = 0; k < kWalkPerLane; ++k) {
        const int j = 64 * k + lane;
        if (k < nk && j < n) stg[j] = tk[k];
    }
}

// The walk over registers filled by walk_load.  A node is acceptable when its
// draft token is the target's choice at its parent (root_want under the
// implicit root) and is not a dead leaf (negative token); that test depends
// only on the node, so it is taken for every node at once, and each step of
// the walk is one ballot per 64 nodes for the current node's lowest-index
// acceptable child.  Writes idx[0, max_depth) (-1 after the path) and returns
// the path length; *next = the target's choice at the last node reached.
__device__ inline int walk_registers(const int (&pk)[kWalkPerLane], const int (&dk)[kWalkPerLane],
                                     const int32_t *stg, int n, int root_want, int max_depth,
                                     int32_t *idx, int *next) {
    const int lane = threadIdx.x & 63;
    const int nk = (n + 63) / 64;  // wave-uniform
    uint32_t okbits = 0;
#pragma unroll
    for (int k = 0; k < kWalkPerLane; ++k) {
        if (k < nk) {
            const int p = pk[k];
            const int want = p == -1 ? root_want : (p >= 0 && p < n ? stg[p] : -1);
            if (dk[k] >= 0 && dk[k] == want) okbits |= 1u << k;
        }
    }
    int cur = -1;
    int len = 0;
    while (len < max_depth) {
        int found = -1;
#pragma unroll
        for (int k = 0; k < kWalkPerLane; ++k) {
            if (k >= nk) break;
            const unsigned long long bal = __ballot(((okbits >> k) & 1u) && pk[k] == cur);
            if (bal) {
                found = 64 * k + __builtin_ctzll(bal);
                break;
            }
        }
        if (found < 0) break;
        if (lane == 0) idx[len] = found;
        ++len;
        cur = found;
    }
    for (int j = len + lane; j < max_depth; j += 64) idx[j] = -1;
    *next = cur < 0 ? root_want : stg[cur];
    return len;
}

// Gathers one KV head's slice of the accepted path's rows into place: row
// P + j receives what row P + sidx[j] held, for j < L.  Sources and
// destinations overlap (a path [0, 2, 5] reads row P + 2 and also writes
// it), so every source row is read into LDS (stage, 2 * max_depth rows)
// before a barrier and only then written; rows already in place are skipped.
// All threads of the workgroup call it; base = the byte offset of row P's
// slice of this head.
template <int ROW_BYTES, int THREADS>
__device__ inline void gather_path(uint8_t *kc, uint8_t *vc, int64_t base, int64_t row_stride,
                                   const int32_t *sidx, int L, int max_depth, uint4 *stage) {
    constexpr int V16 = ROW_BYTES / 16;  // 16-byte vectors per row
    const int tid = threadIdx.x;
    uint4 *sk = stage;
    uint4 *sv = stage + (size_t)max_depth * V16;
    const int work = L * V16;
    for (int e = tid; e < work; e += THREADS) {
        const int j = e / V16, c = e % V16;
        const int64_t off = base + (int64_t)sidx[j] * row_stride + c * 16;
        sk[e] = *reinterpret_cast<const uint4 *>(kc + off);
        sv[e] = *reinterpret_cast<const uint4 *>(vc + off);
    }
    __syncthreads();
    for (int e = tid; e < work; e += THREADS) {
        const int j = e / V16, c = e % V16;
        if (sidx[j] == j) continue;
        const int64_t off = base + (int64_t)j * row_stride + c * 16;
        *reinterpret_cast<uint4 *>(kc + off) = sk[e];
        *reinterpret_cast<uint4 *>(vc + off) = sv[e];
    }
}

}  // namespace tv
