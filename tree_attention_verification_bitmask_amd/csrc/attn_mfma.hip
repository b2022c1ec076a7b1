// tree_attn_verify, MFMA path (bf16 in, fp32 accumulate) for gfx950.
//
// [TSD] = "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
// Tree Attention Accelerate LLM Serving" (llms.blog), section "The Tree
// Attention Mechanism": every node of the flattened tree attends to the whole
// prefix KV cache plus its own ancestors-or-self (parts 1 and 2).
//
// Rows and tiles.  For one request b and KV head g the query rows are the
// (node, head-in-group) pairs r = node * G + j, G = hq / hkv: the G heads that
// share a KV head are stacked so that one K/V stream serves N*G rows.  A
// workgroup takes a tile of 128 rows and one slice of the key axis.  Its eight
// wavefronts form four row groups of 32 rows times two key phases: the two
// waves of a row group take alternate 32-key chunks of the slice, each keeping
// its own online-softmax state, and merge through LDS at the end.
//
// Software pipeline.  Each wave's chunk i goes through S = Q K^T at step i and
// the softmax plus O += P V at step i + 1.  The two waves of a row group share
// a SIMD and order their steps oppositely (products first / softmax first),
// so one keeps the matrix core busy while the other runs the vector ALU.  A
// workgroup barrier separates the steps.
//
// K/V staging.  Chunks of 32 keys are copied HBM -> LDS by the LDS-DMA form of
// the global load (16 bytes per lane, no registers) into two rings of eight
// stages, one for K and one for V.  The K of a chunk is fetched three steps
// before its Q K^T and the V three steps before its P V, so every DMA has
// three steps to land.  The DMA is issued from inline assembly: the compiler
// would otherwise make every LDS read wait for all outstanding DMA, which
// serialises the rings.  The waits are explicit (vmcnt, then the step's
// barrier).  Each 16-byte granule of a cached K/V row lands at an
// XOR-swizzled position in its LDS row so the matrix-operand reads below are
// free of bank conflicts.
//
// Transposed products.  S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = 32 keys
// x 16 channels of K read from LDS, B = Q^T held in registers.  LDS row i of a
// chunk holds key key_of_slot(i), chosen so that in the 32x32 accumulator each
// lane holds one query row and 16 *consecutive* keys: the row max and sum need
// one exchange between the wave halves (v_permlane32_swap).  Then O^T += V^T
// P^T, A = V^T produced from the row-major V chunk by the transposing LDS read
// (ds_read_b64_tr_b16), B = P^T, which is exactly the probabilities the lane
// already holds, packed to bf16.  The O^T accumulator again gives each lane one
// query row, so the online-softmax rescale is lane-local.
//
// Softmax.  Probabilities are 2^((s - m) c) with c = scale * log2(e) and m a
// running reference that is raised only when a chunk's maximum exceeds it by
// more than 8 / c (the weights then stay below 2^8); the accumulators are
// rescaled only then.  The row sum adds the bf16-rounded weights (v_dot2 with
// ones), i.e. exactly the weights the P V product uses.
//
// The ancestor mask is applied per lane, on chunks that reach the tree tail:
// the lane takes the 16 bits of its node's packed row (staged in LDS) that
// cover its 16 keys.  Prefix keys are always visible; keys at or past the end
// of the slice never are (their LDS rows hold a clamped, valid cache row, so
// the P V product never multiplies a zero weight by stale data).
//
// Split key axis.  The host picks `splits` slices of `keys_per_split` keys so
// that the grid fills the chip.  With one slice the kernel writes the
// normalised output; otherwise it writes fp32 partials (unnormalised O, the
// reference m, the sum l) and attn_combine_kernel merges them.
//
// XCD-aware order.  Workgroup ids are dealt round-robin to the 8 XCDs; the
// kernel maps id -> task so that each XCD gets a contiguous block of tasks,
// ordered with the row tiles of one (request, KV head, slice) adjacent, so the
// tiles that read the same K/V run on one XCD and share its L2.
#include "tv_device.h"
#include "tv_launch.h"

#include <stdlib.h>

#include <type_traits>

namespace tv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowGroups = 4;                 // 32-row groups per tile
constexpr int kPhases = kWaves / kRowGroups;  // waves per row group (alternate chunks)
constexpr int kTileRows = 32 * kRowGroups;    // query rows per workgroup
constexpr int kChunk = 32;                    // keys per LDS stage
constexpr int kStages = 8;                    // stages per ring (K ring, V ring)
constexpr int kAhead = 3;                     // steps between a DMA and its use
constexpr int kXcds = 8;
constexpr int kMaxWords = (TV_MAX_NODES + 63) / 64;
constexpr int kAncBytes = kTileRows * kMaxWords * 8;  // packed rows of the tile's nodes
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.f;           // lazy-rescale threshold (log2 units)
static_assert(kPhases == 2, "two key phases");
// K of chunk c lives in K stage c % kStages from step c/2 - kAhead to step c/2;
// V from step c/2 + 1 - kAhead to step c/2 + 1.  Both fit eight stages:
static_assert(kStages >= kPhases * (kAhead + 1), "ring depth");
// The main loop is unrolled by kStages / kPhases steps so that stage indices
// are compile-time constants.
static_assert(kStages == 4 * kPhases, "unroll of the main loop");

template <int D>
struct Geo {
    static constexpr int kRowBytes = 2 * D;                  // one head of one cache row
    static constexpr int kGran = D / 8;                      // 16-byte granules per row
    static constexpr int kHalf = kChunk * kRowBytes;         // K (or V) bytes per chunk
    static constexpr int kDmaPerHalf = kHalf / 1024;         // 1 KB per wave-wide DMA
    static constexpr int kDmaPerWave = kDmaPerHalf / (kWaves / kPhases);  // per chunk half and wave
    static constexpr int kKS = D / 16;                       // k-steps of Q K^T
    static constexpr int kDB = D / 32;                       // 32-channel blocks of O
    static constexpr int kRingBytes = 2 * kStages * kHalf;   // K ring + V ring
    static_assert(kDmaPerWave >= 1 && kDmaPerHalf % (kWaves / kPhases) == 0, "DMA split");
    static_assert(kRowGroups * kDB * 16 * 64 * 4 + kRowGroups * 64 * 8 <= kRingBytes, "merge buffer");
};

// LDS row `slot` (0..31) of a 32-key block holds key key_of_slot(slot): in the
// 32x32 accumulator of S^T, lane half h then holds keys 16h .. 16h+15.
__device__ __forceinline__ int key_of_slot(int slot) {
    return 16 * ((slot >> 2) & 1) + 4 * (slot >> 3) + (slot & 3);
}
// XOR swizzles of the 16-byte granule position within an LDS row.
template <int D>
__device__ __forceinline__ int k_swz(int row) { return row & (Geo<D>::kGran - 1); }
template <int D>
__device__ __forceinline__ int v_swz(int row) { return (4 * row) & (Geo<D>::kGran - 1); }

__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One wave-wide LDS-DMA: every lane copies the 16 bytes at base + voff to
// lds + 16 * lane.  base (a 64-bit pointer) and lds are wave-uniform.  M0
// (the LDS address) is saved and restored around it.
__device__ __forceinline__ void dma16(const char *base, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(base), "s"(lds)
        : "memory");
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N) only.  Inline assembly, so the compiler neither drops
// nor merges it (it does not see the DMA it waits for).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// vmcnt wait allowing n outstanding DMA instructions of this wave, n a
// multiple of PW between 0 and 4 PW.
template <int PW>
__device__ __forceinline__ void wait_dma(int n) {
    if (n >= 4 * PW) wait_vm<4 * PW>();
    else if (n >= 3 * PW) wait_vm<3 * PW>();
    else if (n >= 2 * PW) wait_vm<2 * PW>();
    else if (n >= PW) wait_vm<PW>();
    else wait_vm<0>();
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
    float *ws_o;    // partial O, lane-native layout (see attn_fwd_kernel)
    float2 *ws_ml;  // partial (m, l) per row
    int32_t *err;
};

// Bits e = 0..15 set iff key (key0 + e) is visible to the node whose packed
// ancestor row (in LDS) is `arow`: prefix keys (< P) always, tree key P + j iff
// bit j, nothing at or past `key_hi`.
__device__ __forceinline__ uint32_t visible16(const uint64_t *arow, int words, int key0, int P,
                                              int key_hi) {
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

// Task of workgroup `wid`: (request, KV head, key slice, row tile), XCD-aware.
struct Task {
    int b, g, s, rt;
};
__device__ __forceinline__ bool decode_task(const KParams &p, int wid, Task *t) {
    const int ntasks = p.batch * p.hkv * p.splits * p.row_tiles;
    const int per_xcd = (ntasks + kXcds - 1) / kXcds;
    const int task = (wid % kXcds) * per_xcd + wid / kXcds;
    if (task >= ntasks) return false;
    t->rt = task % p.row_tiles;
    int rest = task / p.row_tiles;
    t->s = rest % p.splits;
    rest /= p.splits;
    t->g = rest % p.hkv;
    t->b = rest / p.hkv;
    return true;
}

// DMA of one half (K or V) of chunk `cidx` of the slice: the four waves of
// key phase cidx & 1 each copy kDmaPerWave KB (part `part` of the half).
// Lane offsets `voff` (bytes from the chunk's first cache row) are
// precomputed; a chunk that runs past k_hi recomputes them with the keys
// clamped to k_hi - 1, so every source row is a valid row of the request.
template <int D>
__device__ __forceinline__ void issue_half(const char *base, int64_t row_stride, int k_lo, int k_hi, int cidx,
                                           bool isv, int part, int lane, const uint32_t *voff,
                                           uint32_t ring_lds) {
    using Gm = Geo<D>;
    const int key0 = k_lo + cidx * kChunk;
    const char *cbase = base + (int64_t)key0 * row_stride;
    const uint32_t lds = ring_lds + (isv ? kStages * Gm::kHalf : 0) + (cidx % kStages) * Gm::kHalf +
                         part * Gm::kDmaPerWave * 1024;
    const bool clamp = key0 + kChunk > k_hi;
#pragma unroll
    for (int i = 0; i < Gm::kDmaPerWave; ++i) {
        uint32_t off = voff[i];
        if (clamp) {
            const int byte = (part * Gm::kDmaPerWave + i) * 1024 + lane * 16;
            const int row = byte / Gm::kRowBytes;
            const int pos = (byte % Gm::kRowBytes) >> 4;
            const int key = isv ? row : key_of_slot(row);
            const int gran = pos ^ (isv ? v_swz<D>(row) : k_swz<D>(row));
            const int kk = min(key0 + key, k_hi - 1) - key0;
            off = (uint32_t)(kk * row_stride) + (uint32_t)(gran << 4);
        }
        dma16(cbase, off, lds + i * 1024);
    }
}

template <int D>
__global__ void __launch_bounds__(kThreads, 1) attn_fwd_kernel(KParams p) {
    using Gm = Geo<D>;
    constexpr int KS = Gm::kKS, DB = Gm::kDB, PW = Gm::kDmaPerWave;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Gm::kRingBytes + kAncBytes];

    Task tk;
    if (!decode_task(p, blockIdx.x, &tk)) return;
    const int b = tk.b, g = tk.g, s = tk.s, rt = tk.rt;

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
    const int node_first = row0 / G;
    const int node_last = (row_end - 1) / G;
    const int key_end = P + node_last + 1;  // tree keys past the tile's last node are never visible
    const int k_lo = s * p.keys_per_split;
    if (k_lo >= key_end) return;
    const int k_hi = min(k_lo + p.keys_per_split, key_end);
    const int nchunks = (k_hi - k_lo + kChunk - 1) / kChunk;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lane = tid & 63;
    const int rg = wave % kRowGroups;
    const int ph = wave / kRowGroups;
    const int col = lane & 31;  // query row within the row group
    const int half = lane >> 5;

    const int64_t row_stride = (int64_t)p.hkv * D * 2;  // bytes per cache row
    const char *kbase = reinterpret_cast<const char *>(p.k) + ks * row_stride + (int64_t)g * D * 2;
    const char *vbase = reinterpret_cast<const char *>(p.v) + ks * row_stride + (int64_t)g * D * 2;
    const uint32_t ring = (uint32_t)(uintptr_t)smem;

    // ---- DMA lane offsets: this wave copies part `rg` of the K and V halves of
    // the chunks of key phase `ph` (chunk-relative source byte offsets).
    uint32_t koffd[PW], voffd[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int byte = (rg * PW + i) * 1024 + lane * 16;
        const int row = byte / Gm::kRowBytes;
        const int pos = (byte % Gm::kRowBytes) >> 4;
        koffd[i] = (uint32_t)(key_of_slot(row) * row_stride) + ((pos ^ k_swz<D>(row)) << 4);
        voffd[i] = (uint32_t)(row * row_stride) + ((pos ^ v_swz<D>(row)) << 4);
    }
    // DMA schedule: at step j (j = -kAhead .. -1 in the prologue) the K of
    // chunks 2 (j + kAhead) + {0, 1} and the V of chunks 2 (j + kAhead - 1) +
    // {0, 1}; this wave copies its part of the chunk of its own phase.
    auto issue_step = [&](int j) {
        const int ck = kPhases * (j + kAhead) + ph;
        if (ck < nchunks)
            issue_half<D>(kbase, row_stride, k_lo, k_hi, ck, false, rg, lane, koffd, ring);
        const int cv = kPhases * (j + kAhead - 1) + ph;
        if (cv >= 0 && cv < nchunks)
            issue_half<D>(vbase, row_stride, k_lo, k_hi, cv, true, rg, lane, voffd, ring);
    };
    auto issued_at = [&](int j) {  // DMA instructions this wave issues at step j
        const int ck = kPhases * (j + kAhead) + ph;
        const int cv = kPhases * (j + kAhead - 1) + ph;
        return PW * ((ck < nchunks ? 1 : 0) + (cv >= 0 && cv < nchunks ? 1 : 0));
    };

    // ---- prologue: start the rings first, so their latency overlaps the loads
    // of Q and of the ancestor rows below.
    for (int j = -kAhead; j < 0; ++j) issue_step(j);

    // ---- this lane's query row -------------------------------------------------
    const int r = row0 + rg * 32 + col;
    const bool row_ok = r < row_end;
    const int node = row_ok ? r / G : node_last;
    const int head = g * G + (row_ok ? r % G : 0);
    const int64_t t = (int64_t)lo + node;
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

    // ---- packed ancestor rows of the tile's nodes -> LDS (only if the slice
    // reaches the tree tail).  Visible to every wave after the first barrier.
    uint64_t *anc_lds = reinterpret_cast<uint64_t *>(smem + Gm::kRingBytes);
    if (k_hi > P) {
        const int cnt = (node_last - node_first + 1) * p.words;
        const uint64_t *src = p.anc + ((int64_t)lo + node_first) * p.words;
        for (int i = tid; i < cnt; i += kThreads) anc_lds[i] = src[i];
    }
    // Make the Q registers live here (the compiler waits for all loads so far,
    // DMA included, once, instead of inside the loop).
#pragma unroll
    for (int k16 = 0; k16 < KS; ++k16) asm volatile("" : "+v"(qb[k16]));

    // ---- per-lane LDS read offsets ----------------------------------------------
    // K (A of S^T): LDS row col, logical granule 2*k16 + half.  The phase's
    // chunks sit in the odd or even stages, hence the ph * kHalf.
    uint32_t koff[KS];
#pragma unroll
    for (int k16 = 0; k16 < KS; ++k16)
        koff[k16] = ph * Gm::kHalf + col * Gm::kRowBytes + (((2 * k16 + half) ^ k_swz<D>(col)) << 4);
    // V (A of O^T via the transposing read): lane l = 16 q + 4 j + rr reads 4
    // channels of key row 16 (q >> 1) + j (+ 4 e + 8 tt), channels
    // 32 db + 16 (q & 1) + 4 rr.
    uint32_t voff[DB];
    {
        const int q = lane >> 4, j = (lane >> 2) & 3, rr = lane & 3;
        const int vrow = 16 * (q >> 1) + j;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int gran = 4 * db + 2 * (q & 1) + (rr >> 1);
            voff[db] = (kStages + ph) * Gm::kHalf + vrow * Gm::kRowBytes + ((gran ^ v_swz<D>(vrow)) << 4) +
                       (rr & 1) * 8;
        }
    }

    f32x16_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    f32x16_t s_new, s_old;
#pragma unroll
    for (int i = 0; i < 16; ++i) s_new[i] = s_old[i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c = p.c;
    const float thr = kRescaleLog2 / c;
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    const uint64_t *arow = anc_lds + (node - node_first) * p.words;

    // ---- main loop ------------------------------------------------------------------
    // Step k: this wave (phase ph) runs Q K^T of its chunk k and the softmax
    // and P V of its chunk k - 1 (its chunk i is chunk 2 i + ph of the slice).
    // Before the barrier every wave waits for the DMA it issued kAhead steps
    // ago (the K of chunks 2k, 2k+1 and the V of chunks 2k-2, 2k-1); after it,
    // it issues the DMA of step k.
    const int my_n = (nchunks + 1 - ph) / 2;
    const int nsteps = (nchunks + 1) / 2 + 1;
    // One step.  U = k % 4 is a compile-time constant (the loop below is
    // unrolled by four), which makes every LDS read offset an immediate: the
    // phase's chunk 2k + ph sits in stage 2 U + ph of the K ring, chunk
    // 2(k-1) + ph in stage 2 ((U + 3) % 4) + ph of the V ring.  s_new / s_old
    // alternate between two register sets.
    auto step = [&](auto U_, int k, f32x16_t &s_new, f32x16_t &s_old) {
        constexpr int U = decltype(U_)::value;
        constexpr uint32_t kst = 2 * U * Gm::kHalf;
        constexpr uint32_t vst = 2 * ((U + 3) & 3) * Gm::kHalf;
        wait_dma<PW>(issued_at(k - 1) + issued_at(k - 2));
        lds_barrier();
        issue_step(k);
        const bool qk = k < my_n;                 // S = Q K^T for chunk k
        const bool sp = k >= 1 && k - 1 < my_n;   // softmax and O += P V for chunk k - 1

        // All LDS operand reads of the step first, so their latency overlaps.
        bf16x8_t va[2][DB], ka[KS];
        if (sp) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint32_t a0 = vst + voff[db] + (8 * tt) * Gm::kRowBytes;
                    const bf16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(smem + a0));
                    const bf16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4_t *)(smem + a0 + 4 * Gm::kRowBytes));
                    va[tt][db] = bf16x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                }
        }
        if (qk) {
#pragma unroll
            for (int k16 = 0; k16 < KS; ++k16) ka[k16] = *reinterpret_cast<const bf16x8_t *>(smem + kst + koff[k16]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (qk) {
#pragma unroll
            for (int e = 0; e < 16; ++e) s_new[e] = 0.f;
#pragma unroll
            for (int k16 = 0; k16 < KS; ++k16)
                s_new = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[k16], qb[k16], s_new, 0, 0, 0);
        }
        if (!sp) return;
        // softmax of chunk k - 1 (its S is s_old), then O += P V
        const int c0 = k_lo + (2 * (k - 1) + ph) * kChunk;
        if (c0 + kChunk > P || c0 + kChunk > k_hi) {
            const uint32_t vis = visible16(arow, p.words, c0 + 16 * half, P, k_hi);
            if (vis != 0xFFFFu) {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (!((vis >> e) & 1u)) s_old[e] = -INFINITY;
            }
        }
        float mx = fmaxf(s_old[0], s_old[1]);
#pragma unroll
        for (int e = 2; e < 16; e += 2) mx = fmaxf(mx, fmaxf(s_old[e], s_old[e + 1]));
        mx = halves_max(mx);
        if (__builtin_amdgcn_ballot_w64(mx > m_run + thr) != 0) {
            const float mn = fmaxf(m_run, mx);
            const float mref = (mn == -INFINITY) ? 0.f : mn;
            const float alpha = __builtin_amdgcn_exp2f((m_run - mref) * c);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
            m_run = mn;
        }
        const float nb = (m_run == -INFINITY) ? 0.f : -m_run * c;
        bf16x8_t pw[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int j2 = 0; j2 < 4; ++j2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s_old[8 * tt + 2 * j2], c, nb));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s_old[8 * tt + 2 * j2 + 1], c, nb));
                bf16x2_t pp;
                pp[0] = (__bf16)p0;
                pp[1] = (__bf16)p1;
                l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
                pw[tt][2 * j2] = pp[0];
                pw[tt][2 * j2 + 1] = pp[1];
            }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[tt][db], pw[tt], oacc[db], 0, 0, 0);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    f32x16_t sa = s_new, sb = s_old;
    for (int k0 = 0; k0 < nsteps; k0 += 4) {
        step(I0{}, k0, sa, sb);
        if (k0 + 1 >= nsteps) break;
        step(I1{}, k0 + 1, sb, sa);
        if (k0 + 2 >= nsteps) break;
        step(I2{}, k0 + 2, sa, sb);
        if (k0 + 3 >= nsteps) break;
        step(I3{}, k0 + 3, sb, sa);
    }

    // ---- merge the two key phases of each row group through LDS ---------------
    l_run = halves_sum(l_run);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // all LDS reads returned
    lds_barrier();
    float *xo = reinterpret_cast<float *>(smem);                                       // [rg][DB*16][64]
    float2 *xml = reinterpret_cast<float2 *>(smem + kRowGroups * DB * 16 * 64 * 4);  // [rg][64]
    if (ph == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) xo[(rg * DB * 16 + db * 16 + i) * 64 + lane] = oacc[db][i];
        xml[rg * 64 + lane] = make_float2(m_run, l_run);
    }
    __syncthreads();
    if (ph == 1) return;
    {
        const float2 o = xml[rg * 64 + lane];
        const float mn = fmaxf(m_run, o.x);
        const float mref = (mn == -INFINITY) ? 0.f : mn;
        const float a0 = __builtin_amdgcn_exp2f((m_run - mref) * c);
        const float a1 = __builtin_amdgcn_exp2f((o.x - mref) * c);
        l_run = l_run * a0 + o.y * a1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                oacc[db][i] = oacc[db][i] * a0 + xo[(rg * DB * 16 + db * 16 + i) * 64 + lane] * a1;
        m_run = mn;
    }

    // ---- epilogue ----------------------------------------------------------------
    if (p.splits == 1) {
        if (!row_ok) return;
        const float inv = 1.f / l_run;
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
        // lane-native partial layout: [tile][split][row group][DB*4 float4][64 lanes]
        const int tile = (b * p.hkv + g) * p.row_tiles + rt;
        const int64_t unit = ((int64_t)tile * p.splits + s) * kRowGroups + rg;
        float4 *po = reinterpret_cast<float4 *>(p.ws_o) + unit * (DB * 4 * 64) + lane;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                po[(db * 4 + i4) * 64] = make_float4(oacc[db][4 * i4 + 0], oacc[db][4 * i4 + 1],
                                                     oacc[db][4 * i4 + 2], oacc[db][4 * i4 + 3]);
        if (half == 0) p.ws_ml[unit * 32 + col] = make_float2(m_run, l_run);
    }
}

// Merge the per-slice partials of one (tile, row group, channel block):
// O = sum_s w_s O_s / sum_s w_s l_s with w_s = 2^((m_s - M) c), M = max_s m_s.
// One wavefront per (tile, row group, 32-channel block); lane layout as the
// partials.
template <int D>
__global__ void __launch_bounds__(256) attn_combine_kernel(KParams p) {
    constexpr int DB = Geo<D>::kDB;
    const int tile = blockIdx.x;
    const int db = blockIdx.y;
    const int rg = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
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
    const int r = row0 + rg * 32 + col;
    if (r >= row_end) return;

    const int64_t base = (int64_t)tile * p.splits;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, p.ws_ml[((base + s) * kRowGroups + rg) * 32 + col].x);
    const float mref = (M == -INFINITY) ? 0.f : M;
    float L = 0.f;
    float4 acc[4];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) acc[i4] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < nsplit; ++s) {
        const int64_t unit = (base + s) * kRowGroups + rg;
        const float2 ml = p.ws_ml[unit * 32 + col];
        const float w = __builtin_amdgcn_exp2f((ml.x - mref) * p.c);
        L = fmaf(w, ml.y, L);
        const float4 *po = reinterpret_cast<const float4 *>(p.ws_o) + unit * (DB * 4 * 64) + db * 4 * 64 + lane;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const float4 o = po[i4 * 64];
            acc[i4].x = fmaf(w, o.x, acc[i4].x);
            acc[i4].y = fmaf(w, o.y, acc[i4].y);
            acc[i4].z = fmaf(w, o.z, acc[i4].z);
            acc[i4].w = fmaf(w, o.w, acc[i4].w);
        }
    }
    const float inv = 1.f / L;
    const int node = r / G;
    const int head = g * G + r % G;
    uint16_t *orow = p.out + (((int64_t)lo + node) * p.hq + head) * D;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + 8 * i4 + 4 * half;
        *reinterpret_cast<uint2 *>(orow + d) = make_uint2(pack_bf16x2(acc[i4].x * inv, acc[i4].y * inv),
                                                          pack_bf16x2(acc[i4].z * inv, acc[i4].w * inv));
    }
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
    // MFMA only where (nodes x GQA group) fills at least one 32-row group
    if (dtype != TV_BF16 || (head_dim != 64 && head_dim != 128) || batch <= 0 || max_nodes * G < 32)
        return plan;
    plan.use = true;
    plan.rows_per_tile = kTileRows;
    plan.row_tiles = (max_nodes * G + kTileRows - 1) / kTileRows;
    const int span = max_prefix + max_nodes;  // longest key axis
    const int chunks = (span + kChunk - 1) / kChunk;
    const long base_tasks = (long)batch * hkv * plan.row_tiles;
    // Fill the chip: one workgroup per CU (256 CUs) for a single request; two
    // rounds for several (ragged) requests, so short ones leave room to
    // balance.  A tuning override (TV_MFMA_SPLITS) may fix the count instead.
    const long target = batch == 1 ? 256 : 512;
    int splits = (int)((target + base_tasks - 1) / base_tasks);
    splits = env_int("TV_MFMA_SPLITS", splits);
    if (splits < 1) splits = 1;
    if (splits > chunks) splits = chunks;
    const int cps = (chunks + splits - 1) / splits;  // chunks per split
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
        hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, p);
        if (plan.splits > 1)
            hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(tiles, Geo<128>::kDB), dim3(256), 0, stream, p);
    } else {
        hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, p);
        if (plan.splits > 1)
            hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(tiles, Geo<64>::kDB), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace tv
