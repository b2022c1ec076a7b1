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
// workgroup takes a tile of 256 rows and one slice of the key axis; each of
// its eight wavefronts owns 32 rows (two per SIMD) and keeps its own
// online-softmax state for them over the whole slice.
//
// K/V staging.  The slice is cut into chunks of 32 keys.  Each chunk's K and
// V are copied HBM -> LDS by the LDS-DMA form of the global load (16 bytes per
// lane, no registers) into two rings of eight stages; the eight waves split a
// chunk's copies between them.  The copy of chunk c is issued at step
// c - kAhead.  The DMA is issued from inline assembly (the compiler would
// otherwise make every LDS read wait for all outstanding DMA) and the waits
// are explicit: before the barrier of step i each wave waits for its own part
// of chunk i + 2, so after the barrier chunk i + 2 is whole in LDS.  Each
// 16-byte granule of a cached K/V row lands at an XOR-swizzled position in its
// LDS row so the matrix-operand reads below are free of bank conflicts.
//
// Ping-pong schedule.  Waves 0-3 (group A) and 4-7 (group B) share the four
// SIMDs, one of each per SIMD.  For chunk j a wave runs a vector phase V(j)
// (the softmax of S(j)) and a matrix phase M(j) (O += P(j) V(j), then
// S(j+1) = Q K(j+1)^T, 16 MFMAs, with the operand registers of the next
// phase refilled from LDS right after each product).  A barrier separates
// the phases, and group B runs one phase behind group A, so on every SIMD one
// wave feeds the matrix core while the other computes exponentials.  The
// operands are read one phase ahead, so LDS latency never stalls a product.
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
// The ancestor mask is applied per lane, on chunks that reach the tree tail
// or the end of the slice: the lane takes the 16 bits of its node's packed
// row (staged in LDS) that cover its 16 keys.  Prefix keys are always
// visible; keys at or past the end of the slice never are (their LDS rows hold
// a clamped, valid cache row, so the P V product never multiplies a zero
// weight by stale data).
//
// Split key axis.  The host picks `splits` slices of `keys_per_split` keys so
// that the grid fills the chip.  With one slice the kernel writes the
// normalised output; otherwise it writes partials (O / l in bf16, with the
// fp32 reference m and sum l) and attn_combine_kernel merges them.
//
// XCD-aware order.  Workgroup ids are dealt round-robin to the 8 XCDs; the
// kernel maps id -> task so that the row tiles of one (slice, request, KV
// head), which read the same K/V, run on one XCD and share its L2, while the
// groups themselves are dealt round-robin over the XCDs, KV head fastest, so
// that ragged requests load every XCD alike (see decode_task).
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
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileRows = 32 * kWaves;  // query rows per workgroup
constexpr int kChunk = 32;              // keys per LDS stage
constexpr int kStages = 8;              // stages per ring (K ring, V ring)
constexpr int kAhead = 6;               // the DMA of chunk c is issued at step c - kAhead
constexpr int kAheadShort = 4;          // the same for slices of at most kShortSlice chunks
constexpr int kShortSlice = 12;
constexpr int kXcds = 8;
constexpr int kMaxWords = (TV_MAX_NODES + 63) / 64;
constexpr int kAncBytes = kTileRows * kMaxWords * 8;  // packed rows of the tile's nodes
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold (log2 units)
// Step i reads K(i+2) and V(i+1); the copy issued at step i overwrites the
// stage of chunk i + kAhead - kStages, whose last read (its V) was at step
// i + kAhead - kStages - 1 <= i - 1.  K(i+2) must have been issued before
// step i, i.e. kAhead >= 3.
static_assert(kAhead >= 3 && kAhead <= kStages, "ring depth");
static_assert(kStages * 2 * 32 * 256 + 256 * 16 * 8 <= 160 * 1024, "K/V rings and ancestor rows fit the 160 KB LDS");

template <int D>
struct Geo {
    static constexpr int kRowBytes = 2 * D;                 // one head of one cache row
    static constexpr int kGran = D / 8;                     // 16-byte granules per row
    static constexpr int kHalf = kChunk * kRowBytes;        // K (or V) bytes per chunk
    static constexpr int kDmaPerHalf = kHalf / 1024;        // 1 KB per wave-wide DMA
    static constexpr int kDmaPerWave = kDmaPerHalf / (kWaves / 2);  // per chunk and wave
    static constexpr int kKS = D / 16;                      // k-steps of Q K^T
    static constexpr int kDB = D / 32;                      // 32-channel blocks of O
    static constexpr int kRingBytes = 2 * kStages * kHalf;  // K ring + V ring
    static_assert(kDmaPerWave >= 1 && kDmaPerHalf % (kWaves / 2) == 0, "DMA split over a wave group");
    // V ring offsets: the lane's base (>= K ring size) lives in a register, the
    // stage and sub-block offsets in the 16-bit immediate of the LDS read.
    static_assert((kStages - 1) * kHalf + 12 * kRowBytes < 65536, "LDS immediate range");
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
// The same with 4 bytes per lane (to lds + 4 * lane).
__device__ __forceinline__ void dma4(const char *base, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, %2\n\t"
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
// Wait until at most PW * clamp(n, 0, CAP) of this wave's DMA instructions
// are outstanding (each chunk costs a wave PW instructions).
template <int PW, int CAP>
__device__ __forceinline__ void wait_chunks(int n) {
    static_assert(CAP >= 0 && CAP <= 4, "wait_chunks covers up to four chunks in flight");
    if (CAP >= 4 && n >= 4) wait_vm<PW * (CAP >= 4 ? 4 : 0)>();
    else if (CAP >= 3 && n >= 3) wait_vm<PW * (CAP >= 3 ? 3 : 0)>();
    else if (CAP >= 2 && n >= 2) wait_vm<PW * (CAP >= 2 ? 2 : 0)>();
    else if (CAP >= 1 && n >= 1) wait_vm<PW * (CAP >= 1 ? 1 : 0)>();
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
    uint2 *ws_o;    // partial O / l as bf16, lane-native layout (see attn_fwd_kernel)
    float2 *ws_ml;  // partial (m, l) per row
    const int32_t *task_table;  // batches: task of each workgroup, longest first (or null)
    int32_t *err;
};

// Sizes of request b, with all four reads issued before any test: a chain of
// tests would make each read wait for the one before (one memory round trip
// each).  ok is false when they disagree with the host's sizes.
struct Req {
    int lo, n, P;
    int64_t ks;
    bool ok;
};
__device__ __forceinline__ Req load_request(const KParams &p, int b) {
    Req r;
    const int c0 = p.cu_nodes[b];
    const int c1 = p.cu_nodes[b + 1];
    r.P = p.prefix_len[b];
    r.ks = p.kv_start[b];
    r.lo = c0;
    r.n = c1 - c0;
    const bool bad = (c0 < 0) | (c1 < c0) | (c1 > p.total_nodes) | (r.n > p.max_nodes) | (r.P < 0) |
                     (r.P > p.max_prefix) | (r.ks < 0) | (r.ks + r.P + r.n > p.kv_rows);
    r.ok = !bad;
    return r;
}

// Bits e = 0..15 set iff key (key0 + e) is visible to the node whose packed
// ancestor row (in LDS) is `arow`: prefix keys (< P) always, tree key P + j iff
// bit j, nothing at or past `key_hi`.
typedef __attribute__((address_space(3))) const uint64_t lds_u64_t;
__device__ __forceinline__ uint32_t visible16(lds_u64_t *arow, int words, int key0, int P, int key_hi) {
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
// A group is the row tiles of one (slice, request, KV head); they read the
// same K/V, so a group stays on one XCD and its tiles take adjacent slots
// there.  Groups are numbered q = (s * batch + b) * hkv + g and dealt
// round-robin to the XCDs (XCD = q mod 8, the hardware's order of workgroup
// ids), so every XCD holds every request's slices in nearly equal shares:
// with 8 KV heads each XCD gets one head of every (slice, request), the same
// work on all eight.  Within an XCD the groups come slice by slice, the full
// first slices before the shorter last ones.
struct Task {
    int b, g, s, rt;
};
__device__ __forceinline__ bool decode_task(const KParams &p, int wid, Task *t) {
    if (p.task_table) {
        // planned order (attn_plan_kernel): task index ((b * hkv + g) * splits
        // + s) * row_tiles + rt, or -1 past the real tasks
        const int task = p.task_table[wid];
        if (task < 0) return false;
        t->rt = task % p.row_tiles;
        int rest = task / p.row_tiles;
        t->s = rest % p.splits;
        rest /= p.splits;
        t->g = rest % p.hkv;
        t->b = rest / p.hkv;
        return true;
    }
    const int ngroups = p.batch * p.hkv * p.splits;
    const int x = wid % kXcds;       // XCD
    const int k = wid / kXcds;       // slot on that XCD
    const int q = x + kXcds * (k / p.row_tiles);
    if (q >= ngroups) return false;
    // Within an XCD the slots go round-robin to its 4 shader engines (8 CUs
    // each) and are dispatched in order, so with 2 or 4 tiles per group the
    // slot number alone would fix the tile each engine gets: the engines given
    // the always-busy first tiles would queue while the others idle on the
    // often-empty last tiles of short requests.  For batches the tile order
    // is rotated by the slot's row of 4, so every engine sees every tile
    // position (one request has no empty tiles and keeps the plain order).
    const int i = k % p.row_tiles;
    t->rt = (p.batch > 1 && 4 % p.row_tiles == 0) ? (i + k / 4) % p.row_tiles : i;
    t->g = q % p.hkv;
    const int rest = q / p.hkv;
    t->b = rest % p.batch;
    t->s = rest / p.batch;
    return true;
}

// AH = copy look-ahead in chunks (AH for long slices, fewer for short ones).
template <int D, int AH>
__global__ void __launch_bounds__(kThreads, 1) attn_fwd_kernel(KParams p) {
    static_assert(AH >= 3 && AH <= kStages && AH - 2 <= 4, "ring depth and counted waits");
    using Gm = Geo<D>;
    constexpr int KS = Gm::kKS, DB = Gm::kDB, PW = Gm::kDmaPerWave;
    constexpr uint32_t kHalf = Gm::kHalf;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Gm::kRingBytes + kAncBytes];

    Task tk;
    if (!decode_task(p, blockIdx.x, &tk)) return;
    const int b = tk.b, g = tk.g, s = tk.s, rt = tk.rt;

    const Req rq = load_request(p, b);
    const int lo = rq.lo, n_nodes = rq.n, P = rq.P;
    const int64_t ks = rq.ks;
    if (!rq.ok) {
        if (g == 0 && rt == 0 && s == 0 && threadIdx.x == 0) report(p.err, TV_DEVERR_BAD_REQUEST, b);
        return;
    }
    const int G = p.hq / p.hkv;
    const int rows_b = n_nodes * G;
    const int row0 = rt * kTileRows;
    if (row0 >= rows_b) return;
    const int row_end = min(rows_b, row0 + kTileRows);
    const int node_first = row0 / G;
    const int node_last = (row_end - 1) / G;
    const int key_end = P + node_last + 1;  // tree keys past the tile's last node are never visible
    const int k_lo = s * p.keys_per_split;
    if (k_lo >= key_end) return;
    const int k_hi = min(k_lo + p.keys_per_split, key_end);
    const int n = (k_hi - k_lo + kChunk - 1) / kChunk;  // chunks of the slice (>= 1)
    // chunks i < c_mask lie wholly in the prefix and below k_hi: no mask
    const int c_mask = max(0, (min(P, k_hi) - k_lo) / kChunk);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lane = tid & 63;
    const int col = lane & 31;  // query row within the wave's 32
    const int half = lane >> 5;

    const int64_t row_stride = (int64_t)p.hkv * D * 2;  // bytes per cache row
    const int64_t chunk_bytes = kChunk * row_stride;
    const char *kbase = reinterpret_cast<const char *>(p.k) + (ks + k_lo) * row_stride + (int64_t)g * D * 2;
    const char *vbase = reinterpret_cast<const char *>(p.v) + (ks + k_lo) * row_stride + (int64_t)g * D * 2;
    const uint32_t ring = (uint32_t)(uintptr_t)smem;

    // ---- DMA role: group A (waves 0 .. kWaves/2 - 1) copies the K half of
    // every chunk, group B the V half; wave w copies parts part0 .. part0 +
    // PW - 1 of its half.  Lane offsets are chunk-relative source bytes; for
    // the last chunk the keys are clamped to the slice, so every source row is
    // a valid row of the request.
    const bool grp_b = wave >= kWaves / 2;
    const bool dv = grp_b;
    const int part0 = (wave % (kWaves / 2)) * PW;
    const char *dbase = dv ? vbase : kbase;
    const uint32_t dlds = ring + (dv ? kStages * kHalf : 0u) + part0 * 1024;
    const int last_keys = (k_hi - k_lo) - (n - 1) * kChunk;  // 1..32
    // Source offset of lane `lane` in copy j of this wave, keys clamped to
    // key_cap (the last chunk passes last_keys - 1, the others 31).
    auto dma_off = [&](int j, int key_cap, int ln) {
        const int byte = (part0 + j) * 1024 + ln * 16;
        const int row = byte / Gm::kRowBytes;
        const int pos = (byte % Gm::kRowBytes) >> 4;
        const int key = dv ? row : key_of_slot(row);
        const int gran = pos ^ (dv ? v_swz<D>(row) : k_swz<D>(row));
        return (uint32_t)(min(key, key_cap) * row_stride) + (uint32_t)(gran << 4);
    };
    const int clamp_c = last_keys < kChunk ? n - 1 : -1;  // the chunk that needs clamping
    uint32_t doff[PW];
#pragma unroll
    for (int j = 0; j < PW; ++j) doff[j] = dma_off(j, kChunk - 1, lane);
    // Copy jj of this wave's part of chunk c into ring stage `stage`.
    auto issue1 = [&](int c, uint32_t stage, int jj) {
        const char *src = dbase + (int64_t)c * chunk_bytes;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(dlds + stage * kHalf + jj * 1024);
        if (c == clamp_c) {
            // (lane made opaque: the clamped offset is formed here instead of
            // being hoisted and kept live across the loop)
            int ln = lane;
            asm volatile("" : "+v"(ln));
            dma16(src, dma_off(jj, last_keys - 1, ln), lds);
        } else {
            dma16(src, doff[jj], lds);
        }
    };
    // Copy chunk c into ring stage `stage`.
    auto issue = [&](int c, uint32_t stage) {
#pragma unroll
        for (int jj = 0; jj < PW; ++jj) issue1(c, stage, jj);
    };

    // ---- prologue --------------------------------------------------------------
    // (1) the packed ancestor rows of the tile's nodes -> LDS, if the slice
    // reaches the tree tail (4 bytes per lane; offsets clamped into the rows).
    uint64_t *anc_lds = reinterpret_cast<uint64_t *>(smem + Gm::kRingBytes);
    if (k_hi > P) {
        const int nbytes = (node_last - node_first + 1) * p.words * 8;
        const char *src = reinterpret_cast<const char *>(p.anc + ((int64_t)lo + node_first) * p.words);
        const int nblk = (nbytes + 255) / 256;
        for (int blk = wave; blk < nblk; blk += kWaves) {
            const uint32_t off = (uint32_t)min(blk * 256 + lane * 4, nbytes - 4);
            dma4(src, off, __builtin_amdgcn_readfirstlane(ring + Gm::kRingBytes + blk * 256));
        }
    }
    // (2) this lane's query row -> registers (asynchronous; waited below).
    const int r = row0 + wave * 32 + col;
    const bool row_ok = r < row_end;
    const bool active = row0 + wave * 32 < row_end;  // wave-uniform: the wave has rows
    const int node = row_ok ? r / G : node_last;      // rows past the tile repeat a valid one
    const int head = g * G + (row_ok ? r % G : 0);
    const int64_t t = (int64_t)lo + node;
    bf16x8_t qb[KS];
    {
        const uint16_t *qrow = p.q + (t * p.hq + head) * D + 8 * half;
#pragma unroll
        for (int k16 = 0; k16 < KS; ++k16)
            asm volatile("global_load_dwordx4 %0, %1, off offset:%2"
                         : "=v"(qb[k16])
                         : "v"(qrow), "n"(32 * k16)
                         : "memory");
    }
    // (3) the first AH chunks.  After the wait everything but chunks
    // 2 .. AH-1 has landed.
#pragma unroll
    for (int c = 0; c < AH; ++c)
        if (c < n) issue(c, c);
    wait_chunks<PW, AH - 2>(min(n, AH) - 2);
#pragma unroll
    for (int k16 = 0; k16 < KS; ++k16) asm volatile("" : "+v"(qb[k16]));
    lds_barrier();

    // ---- per-lane LDS read offsets ----------------------------------------------
    // K (A of S^T): LDS row col, logical granule 2*k16 + half, stored at
    // granule (2*k16 + half) ^ k_swz(col); as a byte offset that is
    // kb + ((32 * k16) ^ kt) (the low bit of the swizzle only flips `half`).
    const uint32_t kt = (uint32_t)(k_swz<D>(col) >> 1) << 5;
    const uint32_t kb = col * Gm::kRowBytes + ((half ^ (k_swz<D>(col) & 1)) << 4);
    // V (A of O^T via the transposing read): lane l = 16 q + 4 j + rr reads 4
    // channels of key row 16 (q >> 1) + j (+ 4 e + 8 tt), channels
    // 32 db + 16 (q & 1) + 4 rr, i.e. logical granule 4 db + 2 (q & 1) +
    // (rr >> 1); the swizzle v_swz(row) is a multiple of 4, so the stored
    // offset is vb + ((64 * db) ^ vt).
    uint32_t vb, vt;
    {
        const int q = lane >> 4, j = (lane >> 2) & 3, rr = lane & 3;
        const int vrow = 16 * (q >> 1) + j;
        vt = (uint32_t)(v_swz<D>(vrow) >> 2) << 6;
        vb = kStages * kHalf + vrow * Gm::kRowBytes + ((2 * (q & 1) + (rr >> 1)) << 4) + (rr & 1) * 8;
    }
    // The swizzle terms are made opaque at each use (empty asm) so that the
    // compiler forms the addresses in the loop (one v_xad each) instead of
    // keeping one hoisted register per address live across the loop.
    // Single operands: K granule pair k16 and the V^T operand (tt, db).
    auto read_k1 = [&](uint32_t base, uint32_t t, int k16) {
        return *reinterpret_cast<const bf16x8_t *>(smem + (((32u * k16) ^ t) + base));
    };
    auto read_v1 = [&](uint32_t base, uint32_t t, int tt, int db) {
        const uint32_t a0 = ((64u * db) ^ t) + base + (8 * tt) * Gm::kRowBytes;
        const bf16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(smem + a0));
        const bf16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(smem + a0 + 4 * Gm::kRowBytes));
        return bf16x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    };
    auto read_k = [&](bf16x8_t(&kk)[KS], uint32_t st) {
        const uint32_t base = kb + st;
        uint32_t t = kt;
        asm volatile("" : "+v"(t));
#pragma unroll
        for (int k16 = 0; k16 < KS; ++k16)
            kk[k16] = *reinterpret_cast<const bf16x8_t *>(smem + (((32u * k16) ^ t) + base));
    };
    auto read_v = [&](bf16x8_t(&vv)[2][DB], uint32_t st) {
        const uint32_t base = vb + st;
        uint32_t t = vt;
        asm volatile("" : "+v"(t));
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint32_t a = ((64u * db) ^ t) + base;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const uint32_t a0 = a + (8 * tt) * Gm::kRowBytes;
                const bf16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(smem + a0));
                const bf16x4_t hi4 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(smem + a0 + 4 * Gm::kRowBytes));
                vv[tt][db] = bf16x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            }
        }
    };

    // ---- ping-pong schedule -------------------------------------------------------
    // Group A = waves 0 .. kWaves/2 - 1, group B = the others; every SIMD holds
    // one wave of each.  For chunk j a wave runs
    //   V(j): the softmax of S(j) -> P(j) (vector work only);
    //   M(j): O += P(j) V(j) and S(j+1) = Q K(j+1)^T (16 products), plus the
    //         reads of V(j+1) and K(j+2) from LDS into registers.
    // V(j) starts with the wave's copies (K for A, V for B) of chunk
    // j + AH: the vector phase has issue slots to spare.
    // Every wave runs V(0) M(0) V(1) M(1) ... with a barrier after each item;
    // group B first passes one barrier alone, so it runs one item behind and
    // on each SIMD one wave feeds the matrix core while the other runs the
    // exponentials.  Barrier 2j+1 starts A's M(j): before it A waits for its
    // part of K(j+2) and B (at the end of its M(j-1)) for its part of V(j+1).
    // A copy issued in V(j) overwrites the stage of chunk j + AH - 8,
    // whose last reads (B's M of chunk j + AH - 9) were consumed at least
    // two items earlier.
    auto copy_ahead = [&](int j) {
        if (j + AH < n) issue(j + AH, (uint32_t)((j + AH) % kStages));
    };
    auto copy_ahead1 = [&](int j, int jj) {
        if (j + AH < n) issue1(j + AH, (uint32_t)((j + AH) % kStages), jj);
    };
    // Waits ahead of the barrier that opens A's M(j) (A: K(j+2)) and the one
    // that opens A's M(j+1) (B, after its M(j): V(j+2)).
    auto wait_before_m = [&](int j) {
        if (!grp_b) wait_chunks<PW, AH - 2>(n - (j + 3));
    };
    auto wait_after_m = [&](int j) {
        if (grp_b) wait_chunks<PW, AH - 2>(n - (j + 3));
    };
    if (!active) {
        // A wave without rows only keeps the copy schedule and the barriers.
        if (grp_b) lds_barrier();
        for (int j = 0; j < n; ++j) {
            copy_ahead(j);
            wait_before_m(j);
            lds_barrier();
            wait_after_m(j);
            lds_barrier();
        }
        if (!grp_b) lds_barrier();
        return;
    }

    f32x16_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    const f32x16_t zero16 = {};
    float m_run = -INFINITY, l_run = 0.f;
    float nb = 0.f;           // -m_ref * c
    const float c = p.c;
    const float thr = kRescaleLog2 / c;
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    lds_u64_t *arow = reinterpret_cast<lds_u64_t *>(
        (uint32_t)(uintptr_t)anc_lds + (uint32_t)((node - node_first) * p.words * 8));

    auto qk = [&](const bf16x8_t(&kk)[KS]) {
        f32x16_t acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[0], qb[0], zero16, 0, 0, 0);
#pragma unroll
        for (int k16 = 1; k16 < KS; ++k16) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[k16], qb[k16], acc, 0, 0, 0);
        return acc;
    };
    // Softmax of chunk i, first part: mask, row max, and (rarely) a raise of
    // the reference m with the rescale of l and O.
    auto prep = [&](f32x16_t &sv, int i) {
        if (i >= c_mask) {
            const uint32_t vis = visible16(arow, p.words, k_lo + i * kChunk + 16 * half, P, k_hi);
            if (vis != 0xFFFFu) {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (!((vis >> e) & 1u)) sv[e] = -INFINITY;
            }
        }
        // row max over the lane's 16 scores as a three-level tree of max3
        const float a0 = fmaxf(fmaxf(sv[0], sv[1]), sv[2]), a1 = fmaxf(fmaxf(sv[3], sv[4]), sv[5]);
        const float a2 = fmaxf(fmaxf(sv[6], sv[7]), sv[8]), a3 = fmaxf(fmaxf(sv[9], sv[10]), sv[11]);
        const float a4 = fmaxf(fmaxf(sv[12], sv[13]), sv[14]);
        const float b0 = fmaxf(fmaxf(a0, a1), a2), b1 = fmaxf(fmaxf(a3, a4), sv[15]);
        const float mx = halves_max(fmaxf(b0, b1));
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
            nb = -mref * c;
        }
    };
    // Second part: the weights 2^(s c - m c), rounded to bf16, and their sum.
    // (Two partial sums halve the dependent chain of the row sum.)
    auto weights = [&](const f32x16_t &sv, bf16x8_t(&pw)[2]) {
        float l0 = 0.f, l1 = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int j2 = 0; j2 < 4; ++j2) {
                const f32x2_t pf = {__builtin_amdgcn_exp2f(fmaf(sv[8 * tt + 2 * j2], c, nb)),
                                    __builtin_amdgcn_exp2f(fmaf(sv[8 * tt + 2 * j2 + 1], c, nb))};
                const bf16x2_t pp = __builtin_convertvector(pf, bf16x2_t);
                if (j2 & 1) l1 = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l1, false);
                else l0 = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l0, false);
                pw[tt][2 * j2] = pp[0];
                pw[tt][2 * j2 + 1] = pp[1];
            }
        }
        l_run += l0 + l1;
    };
    auto pv = [&](const bf16x8_t(&vv)[2][DB], const bf16x8_t(&pw)[2]) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv[tt][db], pw[tt], oacc[db], 0, 0, 0);
    };

    // Prologue products: S(0), and the operands K(1), V(0).
    bf16x8_t kr[KS], vr[2][DB], pw[2];
    read_k(kr, 0);
    f32x16_t sv = qk(kr);
    if (n > 1) read_k(kr, kHalf);
    read_v(vr, 0);
    auto vphase = [&](int j) {
        prep(sv, j);
        weights(sv, pw);
    };
    // M(j): each product is followed by the read that refills the operand
    // registers it consumed (V(j+1) after the P V products, K(j+2) after the
    // Q K^T products), so the reads hide under the matrix core and each
    // operand set stays single.  STEADY: j + 2 < n (both refills exist).
    auto mphase = [&](auto steady_, int j) {
        constexpr bool STEADY = decltype(steady_)::value;
        const bool nx1 = STEADY || j + 1 < n, nx2 = STEADY || j + 2 < n;
        const uint32_t vbase = vb + (uint32_t)((j + 1) % kStages) * kHalf;
        const uint32_t kbase = kb + (uint32_t)((j + 2) % kStages) * kHalf;
        uint32_t vtt = vt, ktt = kt;
        asm volatile("" : "+v"(vtt), "+v"(ktt));
        // The wave feeding the matrix core outranks its SIMD partner (in its
        // softmax phase) for issue, so the products and their operand reads go
        // out back to back; the partner's vector work fills the gaps.
        // Measured: c4 53.4 -> 51.8 us, c5 105.8 -> 101.7 us.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int idx = tt * DB + db;
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[tt][db], pw[tt], oacc[db], 0, 0, 0);
                if (nx1) vr[tt][db] = read_v1(vbase, vtt, tt, db);
                __builtin_amdgcn_sched_barrier(0);
            }
        if (nx1) {
            sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[0], qb[0], zero16, 0, 0, 0);
            if (nx2) kr[0] = read_k1(kbase, ktt, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k16 = 1; k16 < KS; ++k16) {
                sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[k16], qb[k16], sv, 0, 0, 0);
                if (nx2) kr[k16] = read_k1(kbase, ktt, k16);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // Results of the phase are pinned here: register-only work must not
        // drift across the barriers into the other phase.
        asm volatile("" : "+v"(sv));
#pragma unroll
        for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(oacc[db]));
    };
    using Steady = std::true_type;
    using Tail = std::false_type;
    auto vphase_pinned = [&](int j) {
        copy_ahead(j);
        vphase(j);
        asm volatile("" : "+v"(pw[0]), "+v"(pw[1]));
    };
    if (grp_b) lds_barrier();
    int j = 0;
    for (; j < n - 2; ++j) {
        vphase_pinned(j);
        wait_before_m(j);
        lds_barrier();
        mphase(Steady{}, j);
        wait_after_m(j);
        lds_barrier();
    }
    for (; j < n; ++j) {
        vphase_pinned(j);
        lds_barrier();
        mphase(Tail{}, j);
        lds_barrier();
    }
    if (!grp_b) lds_barrier();

    // ---- epilogue ----------------------------------------------------------------
    l_run = halves_sum(l_run);
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
        // Partial of this slice: O / l rounded to bf16 (a convex combination of
        // V rows, so bf16 keeps its range) plus the fp32 (m, l).  Lane-native
        // layout [tile][split][wave][DB*4 x 4 bf16][64 lanes].  A row that sees
        // no key of the slice has l = 0 and stores zeros.  The stores are
        // relaxed atomics at agent scope, which write through this XCD's L2:
        // the merge kernel reads them from another XCD anyway, and the end of
        // this kernel then has no dirty partials left to write back
        // (measured: 1.5 us less per call at 240 workgroups).
        const int tile = (b * p.hkv + g) * p.row_tiles + rt;
        const int64_t unit = ((int64_t)tile * p.splits + s) * kWaves + wave;
        uint2 *po = p.ws_o + unit * (DB * 4 * 64) + lane;
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const uint64_t w =
                    (uint64_t)pack_bf16x2(oacc[db][4 * i4 + 0] * inv, oacc[db][4 * i4 + 1] * inv) |
                    ((uint64_t)pack_bf16x2(oacc[db][4 * i4 + 2] * inv, oacc[db][4 * i4 + 3] * inv) << 32);
                __hip_atomic_store(reinterpret_cast<uint64_t *>(po + (db * 4 + i4) * 64), w, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        if (half == 0) {
            const uint64_t w = (uint64_t)__float_as_uint(m_run) | ((uint64_t)__float_as_uint(l_run) << 32);
            __hip_atomic_store(reinterpret_cast<uint64_t *>(p.ws_ml + unit * 32 + col), w, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Merge the per-slice partials of one row of one (tile, 32-row group,
// channels): O = sum_s w_s O_s / sum_s w_s l_s with w_s = 2^((m_s - M) c),
// M = max_s m_s.  One wavefront per (tile, row group, 32-channel block, I4W of
// the 4 float4 slots), four per workgroup; lane layout as the partials (lane
// half h holds channels 32 db + 8 i4 + 4 h .. +3 of row col).  The slices are
// taken in batches whose loads are all issued before any is used, so a batch
// costs one memory round trip; a batch loads only the slices that exist.  With
// few slices (I4W = 4) a wave merges all four slots: four times fewer waves,
// each with four times the loads in flight.
constexpr int kCombineWaves = 4;
template <int D, int I4W>
__global__ void __launch_bounds__(64 * kCombineWaves) attn_combine_kernel(KParams p) {
    constexpr int DB = Geo<D>::kDB;
    constexpr int kGroups = 4 / I4W;                 // waves per (tile, row group, channel block)
    constexpr int kBatch = I4W == 1 ? 16 : 8;        // slices per batch
    // (wave-uniform: the request's sizes then come by scalar loads, which
    // complete independently of the partials' vector loads)
    const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * kCombineWaves + (threadIdx.x >> 6));
    const int i4b = (gw % kGroups) * I4W;
    const int db = (gw / kGroups) % DB;
    const int rg = (gw / (kGroups * DB)) % kWaves;
    const int tile = gw / (kGroups * DB * kWaves);
    if (tile >= p.batch * p.hkv * p.row_tiles) return;
    const int lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int rt = tile % p.row_tiles;
    const int g = (tile / p.row_tiles) % p.hkv;
    const int b = tile / (p.row_tiles * p.hkv);

    // The partials' addresses depend only on (tile, slice, lane), so for one
    // request the first batch is loaded before the request's sizes arrive: the
    // two memory round trips overlap.  Slices the request does not have were never written and
    // hold arbitrary bits; they are skipped by branches below, never scaled by
    // zero (0 * NaN would poison the sum).
    const int64_t base = (int64_t)tile * p.splits;
    const float2 *ml = p.ws_ml + (base * kWaves + rg) * 32 + col;
    const uint2 *po = p.ws_o + (base * kWaves + rg) * (DB * 4 * 64) + (db * 4 + i4b) * 64 + lane;
    constexpr int64_t kMlStride = kWaves * 32;                    // per slice
    constexpr int64_t kOStride = (int64_t)kWaves * DB * 4 * 64;   // per slice
    float2 m_l[kBatch];
    uint2 o[kBatch][I4W];
    // (one request: every tile has nearly all slices, so the early loads are
    // nearly all used; in a ragged batch short requests have few slices, and
    // the loads wait for the sizes instead)
    const int nb0 = p.batch == 1 ? min(kBatch, p.splits) : 0;  // wave-uniform
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        m_l[u] = u < nb0 ? ml[u * kMlStride] : make_float2(-INFINITY, 0.f);
#pragma unroll
        for (int ii = 0; ii < I4W; ++ii) o[u][ii] = u < nb0 ? po[u * kOStride + ii * 64] : make_uint2(0u, 0u);
    }

    const Req rq = load_request(p, b);
    if (!rq.ok) return;
    const int lo = rq.lo, n = rq.n, P = rq.P;
    const int G = p.hq / p.hkv;
    const int rows_b = n * G;
    const int row0 = rt * kTileRows;
    if (row0 + rg * 32 >= rows_b) return;  // (wave-uniform) no rows in this group
    const int row_end = min(rows_b, row0 + kTileRows);
    const int key_end = P + (row_end - 1) / G + 1;
    const int nsplit = min(p.splits, (key_end + p.keys_per_split - 1) / p.keys_per_split);
    const int r = row0 + rg * 32 + col;

    float M = -INFINITY, L = 0.f;
    float4 acc[I4W];
#pragma unroll
    for (int ii = 0; ii < I4W; ++ii) acc[ii] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
        const int nb = min(kBatch, nsplit - s0);  // wave-uniform
        if (s0 > 0 || nb0 == 0) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                // slices past the end issue no load (a uniform branch)
                if (u < nb) {
                    m_l[u] = ml[(s0 + u) * kMlStride];
#pragma unroll
                    for (int ii = 0; ii < I4W; ++ii) o[u][ii] = po[(s0 + u) * kOStride + ii * 64];
                }
            }
        }
        float mb = M;
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (u < nb) mb = fmaxf(mb, m_l[u].x);
        const float mref = (mb == -INFINITY) ? 0.f : mb;
        const float a = __builtin_amdgcn_exp2f((M - mref) * p.c);  // 0 when M = -inf
        L *= a;
#pragma unroll
        for (int ii = 0; ii < I4W; ++ii) {
            acc[ii].x *= a;
            acc[ii].y *= a;
            acc[ii].z *= a;
            acc[ii].w *= a;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (u < nb) {
                // slice weight times its sum: the partial holds O / l
                const float wl = __builtin_amdgcn_exp2f((m_l[u].x - mref) * p.c) * m_l[u].y;
                L += wl;
#pragma unroll
                for (int ii = 0; ii < I4W; ++ii) {
                    acc[ii].x = fmaf(wl, bf16_lo(o[u][ii].x), acc[ii].x);
                    acc[ii].y = fmaf(wl, bf16_hi(o[u][ii].x), acc[ii].y);
                    acc[ii].z = fmaf(wl, bf16_lo(o[u][ii].y), acc[ii].z);
                    acc[ii].w = fmaf(wl, bf16_hi(o[u][ii].y), acc[ii].w);
                }
            }
        }
        M = mb;
    }
    if (r >= row_end) return;
    const float inv = 1.f / L;
    const int node = r / G;
    const int head = g * G + r % G;
    uint16_t *orow = p.out + (((int64_t)lo + node) * p.hq + head) * D;
#pragma unroll
    for (int ii = 0; ii < I4W; ++ii) {
        const int d = db * 32 + 8 * (i4b + ii) + 4 * half;
        *reinterpret_cast<uint2 *>(orow + d) = make_uint2(pack_bf16x2(acc[ii].x * inv, acc[ii].y * inv),
                                                          pack_bf16x2(acc[ii].z * inv, acc[ii].w * inv));
    }
}

// Task plan for batches.  The static order cannot know the requests' sizes,
// and within an XCD the slots are dispatched in order to its shader engines,
// so a long slice behind a queue of short ones finishes late.  One workgroup
// reads every request's sizes, gives each group (request, KV head, slice) the
// chunk count of its longest row tile by the attention kernel's own rules
// (0 = every tile would exit at once), and counting-sorts the non-empty groups
// longest first.  Group k of that order takes workgroup ids
// (k / 8) * 8 * row_tiles + 8 i + k % 8 for its tiles i: consecutive groups on
// consecutive XCDs, and the tiles of one group, which read the same K/V, on
// one XCD in adjacent slots (sharing its L2).  Empty tiles and the padding
// hold -1.  Groups of equal length land in any order: each task writes its
// own partial slot, so the results do not depend on it.  Invalid requests are
// reported here, since no workgroup is planned for them.
constexpr int kPlanThreads = 1024;
constexpr int kPlanBins = 4096;     // chunk counts 1 .. kPlanBins - 1
constexpr int kPlanMaxTasks = 65536;

__device__ __forceinline__ int tile_chunks(const KParams &p, const Req &rq, int s, int rt) {
    if (!rq.ok) return 0;
    const int G = p.hq / p.hkv;
    const int rows_b = rq.n * G;
    const int row0 = rt * kTileRows;
    if (row0 >= rows_b) return 0;
    const int row_end = min(rows_b, row0 + kTileRows);
    const int key_end = rq.P + (row_end - 1) / G + 1;
    const int k_lo = s * p.keys_per_split;
    if (k_lo >= key_end) return 0;
    const int k_hi = min(k_lo + p.keys_per_split, key_end);
    return (k_hi - k_lo + kChunk - 1) / kChunk;
}

// Group q = (b * hkv + g) * splits + s: its longest tile's chunk count.
__device__ __forceinline__ int group_chunks(const KParams &p, int q) {
    const int s = q % p.splits;
    const int b = q / p.splits / p.hkv;
    const Req rq = load_request(p, b);
    int len = 0;
    for (int rt = 0; rt < p.row_tiles; ++rt) len = max(len, tile_chunks(p, rq, s, rt));
    return len;
}

__global__ void __launch_bounds__(kPlanThreads) attn_plan_kernel(KParams p, int ngroups, int nslots,
                                                                  int32_t *__restrict__ table) {
    __shared__ int cnt[kPlanBins];
    __shared__ int wsum[kPlanThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int R = p.row_tiles;
    for (int i = tid; i < kPlanBins; i += kPlanThreads) cnt[i] = 0;
    for (int b = tid; b < p.batch; b += kPlanThreads)
        if (!load_request(p, b).ok) report(p.err, TV_DEVERR_BAD_REQUEST, b);
    for (int i = tid; i < nslots; i += kPlanThreads) table[i] = -1;
    __syncthreads();
    for (int q = tid; q < ngroups; q += kPlanThreads) {
        const int len = group_chunks(p, q);
        if (len > 0) atomicAdd(&cnt[len], 1);
    }
    __syncthreads();
    // start of each length's run, longest first: thread tid owns the bins of
    // lengths kPlanBins - 1 - (4 tid .. 4 tid + 3)
    constexpr int kPer = kPlanBins / kPlanThreads;
    int v[kPer];
    int own = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        v[e] = cnt[kPlanBins - 1 - (kPer * tid + e)];
        own += v[e];
    }
    int incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < kPlanThreads / 64; ++w) before += w < wv ? wsum[w] : 0;
    int run = before + incl - own;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        cnt[kPlanBins - 1 - (kPer * tid + e)] = run;
        run += v[e];
    }
    __syncthreads();
    for (int q = tid; q < ngroups; q += kPlanThreads) {
        const int len = group_chunks(p, q);
        if (len <= 0) continue;
        const int k = atomicAdd(&cnt[len], 1);  // rank of the group, longest first
        const int s = q % p.splits;
        const int b = q / p.splits / p.hkv;
        const Req rq = load_request(p, b);
        const int m = k / kXcds;  // the group's rank on its XCD
        const int base = m * kXcds * R + k % kXcds;
        // tile rt goes to slot i of the group, rotated by the slot's row of 4
        // as in the static order, so that every shader engine gets first and
        // last tiles alike
        const int rot = (4 % R == 0) ? (m * R) / 4 : 0;
        for (int rt = 0; rt < R; ++rt) {
            const int i = ((rt - rot) % R + R) % R;
            if (tile_chunks(p, rq, s, rt) > 0) table[base + kXcds * i] = q * R + rt;
        }
    }
}

}  // namespace

MfmaPlan plan_attn_mfma(int batch, int total_nodes, int max_nodes, int max_prefix, int hq, int hkv,
                        int head_dim, tv_dtype dtype, const tv_attn_plan_override *ov) {
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
    // Fill the chip: one workgroup per CU (256 CUs) for a single request.
    // Batches that the planner can order take about four rounds of short
    // slices (8 at c5); otherwise about two and a half in the static order,
    // so short requests leave room to balance.  The override (tuning and
    // tests) may fix the slice count or the batch order instead.
    const long planned = (long)batch * hkv * plan.row_tiles;  // tasks per slice
    const int order = ov ? ov->order : TV_ORDER_AUTO;
    const bool can_plan = batch > 1 && order != TV_ORDER_STATIC;
    const long target = batch == 1 ? 256 : (can_plan ? 1024 : 640);
    int splits = (int)((target + base_tasks - 1) / base_tasks);
    if (ov && ov->splits > 0) splits = ov->splits;
    if (splits < 1) splits = 1;
    if (splits > chunks) splits = chunks;
    const int cps = (chunks + splits - 1) / splits;  // chunks per split
    plan.keys_per_split = cps * kChunk;
    plan.splits = (chunks + cps - 1) / cps;
    if (plan.splits > 1) {
        const size_t rows = (size_t)base_tasks * plan.splits * kTileRows;
        plan.ws_bytes = rows * head_dim * sizeof(uint16_t);
        plan.ws_bytes = (plan.ws_bytes + 255) & ~(size_t)255;
        plan.ws_bytes += rows * sizeof(float2);
        const long ntasks = planned * plan.splits;
        if (can_plan && ntasks <= kPlanMaxTasks && cps < kPlanBins) {
            const long ngroups = (long)batch * hkv * plan.splits;
            plan.table = true;
            plan.table_slots = (int)((ngroups + kXcds - 1) / kXcds * kXcds * plan.row_tiles);
            plan.table_off = (plan.ws_bytes + 255) & ~(size_t)255;
            plan.ws_bytes = plan.table_off + (size_t)plan.table_slots * sizeof(int32_t);
        }
    }
    return plan;
}

int attn_mfma_lookahead(const MfmaPlan &plan) {
    return plan.keys_per_split / kChunk <= kShortSlice ? kAheadShort : kAhead;
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
    p.task_table = nullptr;
    if (plan.splits > 1) {
        const size_t rows = (size_t)a.batch * a.hkv * plan.row_tiles * plan.splits * kTileRows;
        size_t off = rows * a.head_dim * sizeof(uint16_t);
        off = (off + 255) & ~(size_t)255;
        p.ws_o = (uint2 *)workspace;
        p.ws_ml = (float2 *)((char *)workspace + off);
    }
    const long ngroups = (long)a.batch * a.hkv * plan.splits;
    long grid = ((ngroups + kXcds - 1) / kXcds) * plan.row_tiles * kXcds;
    if (plan.table) {
        int32_t *table = (int32_t *)((char *)workspace + plan.table_off);
        const int ngroups_i = a.batch * a.hkv * plan.splits;
        hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p, ngroups_i,
                           plan.table_slots, table);
        p.task_table = table;
        grid = plan.table_slots;
    }
    const long tiles = (long)a.batch * a.hkv * plan.row_tiles;
    // few slices: one merge wave covers all four float4 slots of its channels
    const bool wide = plan.splits <= 8;
    // short slices: the prologue outweighs the loop, so fewer chunks are
    // copied ahead of the first barrier
    const bool short_slices = attn_mfma_lookahead(plan) == kAheadShort;
    const long cwaves = tiles * kWaves * (a.head_dim / 32) * (wide ? 1 : 4);
    const long cblocks = (cwaves + kCombineWaves - 1) / kCombineWaves;
    if (a.head_dim == 128) {
        if (short_slices)
            hipLaunchKernelGGL((attn_fwd_kernel<128, kAheadShort>), dim3(grid), dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((attn_fwd_kernel<128, kAhead>), dim3(grid), dim3(kThreads), 0, stream, p);
        if (plan.splits > 1 && wide)
            hipLaunchKernelGGL((attn_combine_kernel<128, 4>), dim3(cblocks), dim3(64 * kCombineWaves), 0, stream, p);
        else if (plan.splits > 1)
            hipLaunchKernelGGL((attn_combine_kernel<128, 1>), dim3(cblocks), dim3(64 * kCombineWaves), 0, stream, p);
    } else {
        if (short_slices)
            hipLaunchKernelGGL((attn_fwd_kernel<64, kAheadShort>), dim3(grid), dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((attn_fwd_kernel<64, kAhead>), dim3(grid), dim3(kThreads), 0, stream, p);
        if (plan.splits > 1 && wide)
            hipLaunchKernelGGL((attn_combine_kernel<64, 4>), dim3(cblocks), dim3(64 * kCombineWaves), 0, stream, p);
        else if (plan.splits > 1)
            hipLaunchKernelGGL((attn_combine_kernel<64, 1>), dim3(cblocks), dim3(64 * kCombineWaves), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace tv
