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
// workgroup of NW wavefronts (4 or 8) takes a tile of 32 * NW rows and one
// slice of the key axis; each wavefront owns 32 rows and keeps its own
// online-softmax state for them over the whole slice.
//
// K/V staging.  The slice is cut into chunks of 32 keys.  Each chunk's K and
// V are copied HBM -> LDS by the LDS-DMA form of the global load (16 bytes per
// lane, no registers) into two rings of eight stages; the waves split a
// chunk's copies between them.  The copy of chunk c is issued at step
// c - AH.  The DMA is issued from inline assembly (the compiler would
// otherwise make every LDS read wait for all outstanding DMA) and the waits
// are explicit: before the barrier that opens step j each wave waits for its
// own part of chunk j + 2, so after the barrier chunk j + 2 is whole in LDS.
// Each 16-byte granule of a cached K/V row lands at an XOR-swizzled position
// in its LDS row so the matrix-operand reads below are free of bank conflicts.
//
// Per-wave software pipeline.  Step j of a wavefront issues, in one scheduled
// block, the products O += P(j-1) V(j-1) and S(j+1) = Q K(j+1)^T (16 MFMAs at
// head_dim 128) and, interleaved with them, the whole softmax of S(j), which
// the previous step produced: the matrix core runs while the same wave's
// vector unit computes exponentials.  (Measured on gfx950: a wave overlaps its
// own MFMAs with its own vector work almost completely, while a wave that only
// issues MFMAs next to one that only issues vector work on the same SIMD
// does not.)  Each product is followed by the LDS read that refills the
// operand registers it consumed (V(j) after the P V products, K(j+2) after
// the Q K^T products), so the reads have a whole step to land.  One barrier
// per step guards the copy ring.
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
// Softmax.  Scores are kept in log2 units: Q is multiplied by c = scale *
// log2(e) once (and rounded to bf16 again), and the Q K^T accumulator starts
// from -M, M a running reference per row, so a weight is a bare 2^x of the
// product's output (one exponential per score, no other arithmetic).  M is
// raised only when a chunk's maximum exceeds it by more than 8 (the weights
// then stay below 2^8); the accumulators are rescaled only then.  The weights
// of chunk j are computed with the reference in force before chunk j, in
// parallel with its row maximum; in the rare step whose maximum raises the
// reference they are computed again and the scores already formed for the
// next chunk are shifted to the new reference (so nothing waits for the
// maximum in the common case).  The row sum adds the bf16-rounded weights
// (v_dot2 with ones), i.e. exactly the weights the P V product uses.
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

#include <type_traits>

namespace tv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kChunk = 32;              // keys per LDS stage
constexpr int kStages = 8;              // stages per ring (K ring, V ring)
constexpr int kBarrierPeriod = 2;       // steps between the barriers that guard the copy ring
constexpr int kAhead = 5;               // chunks j + kAhead .. j + kAhead + 1 are copied at step j
constexpr int kAheadShort = 4;          // the same for slices of at most kShortSlice chunks
constexpr int kShortSlice = 12;
constexpr int kMinSliceChunks = 5;      // fewest chunks per key-axis slice the plan picks
constexpr int kXcds = 8;
constexpr int kMaxTileRows = 256;
constexpr int kMaxWords = (TV_MAX_NODES + 63) / 64;
constexpr int kAncBytes = kMaxTileRows * kMaxWords * 8;  // packed rows of the tile's nodes
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold (log2 units)
// Ring safety, with BP = kBarrierPeriod and barriers at the steps j = 0, BP,
// 2 BP, ...: step j reads chunks j - 1, j and j + 1, so the last read of
// chunk c is in step c + 1.  The copies issued at the barrier of step j
// (chunks j + AH .. j + AH + BP - 1) overwrite the stages of chunks
// j + AH - 8 .. j + AH + BP - 9, last read in step j + AH + BP - 8, which
// every wave has finished at that barrier when AH + BP <= 7.  Between two
// barriers the waves read chunks up to j + BP, which must have been copied
// at the previous barrier: AH >= BP + 1.
static_assert(kAhead + kBarrierPeriod <= 7 && kAheadShort >= kBarrierPeriod + 1, "ring depth");
static_assert(kStages * 2 * 32 * 256 + kAncBytes <= 160 * 1024, "K/V rings and ancestor rows fit the 160 KB LDS");

template <int D, int NW, int RB>
struct Geo {
    static constexpr int kRowBytes = 2 * D;                 // one head of one cache row
    static constexpr int kGran = D / 8;                     // 16-byte granules per row
    static constexpr int kHalf = kChunk * kRowBytes;        // K (or V) bytes per chunk
    static constexpr int kDmaPerHalf = kHalf / 1024;        // 1 KB per wave-wide DMA
    static constexpr int kDmaPerWave = 2 * kDmaPerHalf / NW;  // per chunk and wave (one half only)
    static constexpr int kKS = D / 16;                      // k-steps of Q K^T
    static constexpr int kDB = D / 32;                      // 32-channel blocks of O
    static constexpr int kRingBytes = 2 * kStages * kHalf;  // K ring + V ring
    static constexpr int kTileRows = 32 * NW * RB;  // RB blocks of 32 rows per wave
    static constexpr int kRowsPerDma = 1024 / kRowBytes;   // cache rows one wave-wide copy covers
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    static_assert(RB == 1 || RB == 2, "one or two 32-row blocks per wave");
    static_assert(kTileRows <= kMaxTileRows, "ancestor rows of the tile fit their LDS area");
    static_assert(kDmaPerWave >= 1 && kDmaPerHalf % kDmaPerWave == 0, "DMA split over half the waves");
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
__device__ __forceinline__ int k_swz(int row) { return row & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int v_swz(int row) { return (4 * row) & (D / 8 - 1); }

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
// The same from a per-lane 64-bit address.
__device__ __forceinline__ void dma16_at(const char *addr, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(addr), "s"(lds)
        : "memory");
}
// The same with 4 bytes per lane (to lds + 4 * lane).
__device__ __forceinline__ void dma4(const char *base_in, uint32_t voff, uint32_t lds) {
    // (the base is wave-uniform; said explicitly, so that it stays in scalar
    // registers whatever the compiler's uniformity analysis concludes)
    const uint64_t bu = (uint64_t)(uintptr_t)base_in;
    const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)bu);
    const uint32_t bhi = __builtin_amdgcn_readfirstlane((uint32_t)(bu >> 32));
    const char *base = (const char *)(uintptr_t)(((uint64_t)bhi << 32) | blo);
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
    static_assert(CAP >= 0 && CAP <= 6 && PW * CAP < 64, "wait_chunks covers up to six chunks in flight");
    if (CAP >= 6 && n >= 6) wait_vm<PW * (CAP >= 6 ? 6 : 0)>();
    else if (CAP >= 5 && n >= 5) wait_vm<PW * (CAP >= 5 ? 5 : 0)>();
    else if (CAP >= 4 && n >= 4) wait_vm<PW * (CAP >= 4 ? 4 : 0)>();
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
    int rgroups, tile_rows;  // 32-row groups per tile, query rows per tile (32 * rgroups)
    int row_tiles, splits, keys_per_split;
    float c;  // scale * log2(e)
    uint16_t *out;
    uint2 *ws_o;    // partial O / l as bf16, lane-native layout (see attn_fwd_kernel)
    float2 *ws_ml;  // partial (m, l) per row
    const int32_t *task_table;  // batches: task of each workgroup, longest first (or null)
    int32_t *err;
    const int32_t *table;    // token table [batch, tstride]: cache row of each key position (or null)
    int64_t tstride;
    int kvr32;               // min(kv_rows, INT32_MAX): bound of a table entry
    const float2 *rope_cs;   // (cos, sin) [T, D/2] to rotate q at load (or null)
    // balanced order (attn_bal_plan_kernel), else null: each workgroup's
    // {first piece, count}; the pieces {tile, first chunk, end chunk, partial
    // slot or -1}; each (request, KV head)'s {first partial, count}
    const int2 *bal_wg;
    const int4 *bal_piece;
    const int2 *bal_group;
    int bal_slots;  // entries of bal_piece, and partial slots (the bound every index is checked against)
    // 1: the static order with a multiple of 8 KV heads, where every slice of
    // KV head g ran on XCD g mod 8; the merge then takes head g's tiles on
    // that XCD too, so it reads the partials where they were written
    int combine_xcd;
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
    r.ks = p.table ? 0 : p.kv_start[b];
    r.lo = c0;
    r.n = c1 - c0;
    // through a token table the request's positions must fit its table row;
    // otherwise its rows must fit the cache
    const bool rows_bad = p.table ? ((int64_t)r.P + r.n > p.tstride) : ((r.ks < 0) | (r.ks + r.P + r.n > p.kv_rows));
    const bool bad = (c0 < 0) | (c1 < c0) | (c1 > p.total_nodes) | (r.n > p.max_nodes) | (r.P < 0) |
                     (r.P > p.max_prefix) | rows_bad;
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

// Rows per row tile for a request of rows_b query rows and tiles of at most TR
// rows: the rows are spread evenly over its ceil(rows_b / TR) tiles, in whole
// 32-row blocks, so the tiles of one key range carry equal work and keep in
// step (sharing the K/V in their XCD's L2) instead of full tiles and a short
// last one.
__device__ __forceinline__ int tile_span(int rows_b, int TR) {
    if (rows_b <= 0) return TR;
    const int R = (rows_b + TR - 1) / TR;
    const int per = (rows_b + R - 1) / R;
    return (per + 31) & ~31;
}

// One piece of work for a workgroup: row tile rt of (request b, KV head g)
// over the keys [k_lo, k_lo + k_span), clipped to the keys the tile's nodes
// can see.  The result goes to the output (pslot < 0) or, normalised by its
// own sum, to partial slot pslot with its (m, l) for the merge kernel.
struct Piece {
    int b, g, rt, k_lo, k_span;
    int64_t pslot;
    bool report_bad;     // the piece that reports an invalid request b
    bool empty_partial;  // a piece with no visible key still writes its partial (an empty one)
};

// The partial of a piece that sees no key of the tile: (m, l) = (-inf, 0) and
// zero O for every row, so a merge that reads it adds nothing.
template <int D, int NW, int RB>
__device__ __forceinline__ void store_empty_partial(const KParams &p, int64_t pslot) {
    constexpr int DB = D / 32;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int64_t unit = pslot * (NW * RB) + wave * RB + rb;
        uint2 *po = p.ws_o + unit * (DB * 4 * 64) + lane;
#pragma unroll
        for (int i = 0; i < DB * 4; ++i)
            __hip_atomic_store(reinterpret_cast<uint64_t *>(po + i * 64), 0ull, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        if (lane < 32) {
            const uint64_t w = (uint64_t)__float_as_uint(-INFINITY);
            __hip_atomic_store(reinterpret_cast<uint64_t *>(p.ws_ml + unit * 32 + lane), w, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// NW = waves per workgroup; RB = 32-row blocks per wave (two blocks share
// every K and V operand read from LDS, halving LDS and L2 traffic per
// product); AH = copy look-ahead in chunks (AH for long slices, fewer for
// short ones); PAGED: K/V rows through the token table.  `smem` is the
// workgroup's LDS (K/V rings, then the ancestor rows); every wave of the
// workgroup runs the piece (the waves without rows keep the copy schedule).
template <int D, int NW, int RB, int AH, bool PAGED>
__device__ __attribute__((always_inline)) inline void attn_piece(const KParams &p, unsigned char *smem,
                                                                 const Piece &pc, int tid) {
    using Gm = Geo<D, NW, RB>;
    constexpr int KS = Gm::kKS, DB = Gm::kDB, PW = Gm::kDmaPerWave, TR = Gm::kTileRows;
    constexpr uint32_t kHalf = Gm::kHalf;
    constexpr int BP = kBarrierPeriod;
    static_assert(AH >= BP + 1 && AH + BP <= 7, "ring safety");
    const int b = pc.b, g = pc.g, rt = pc.rt;

    const Req rq = load_request(p, b);
    const int lo = rq.lo, n_nodes = rq.n, P = rq.P;
    const int64_t ks = rq.ks;
    if (!rq.ok) {
        if (pc.report_bad && threadIdx.x == 0) report(p.err, TV_DEVERR_BAD_REQUEST, b);
        return;
    }
    const int G = p.hq / p.hkv;
    const int rows_b = n_nodes * G;
    const int span = tile_span(rows_b, TR);
    const int row0 = rt * span;
    if (row0 >= rows_b) return;
    const int row_end = min(rows_b, row0 + span);
    const int node_first = row0 / G;
    const int node_last = (row_end - 1) / G;
    const int key_end = P + node_last + 1;  // tree keys past the tile's last node are never visible
    const int k_lo = pc.k_lo;
    if (k_lo >= key_end) {
        if (pc.empty_partial && pc.pslot >= 0) store_empty_partial<D, NW, RB>(p, pc.pslot);
        return;
    }
    const int k_hi = min(k_lo + pc.k_span, key_end);
    const int n = (k_hi - k_lo + kChunk - 1) / kChunk;  // chunks of the slice (>= 1)
    // chunks i < c_mask lie wholly in the prefix and below k_hi: no mask
    const int c_mask = max(0, (min(P, k_hi) - k_lo) / kChunk);

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lane = tid & 63;
    const int col = lane & 31;  // query row within the wave's 32
    const int half = lane >> 5;

    const int64_t row_stride = (int64_t)p.hkv * D * 2;  // bytes per cache row
    const int64_t chunk_bytes = kChunk * row_stride;
    // (through a token table a chunk's rows are anywhere: the bases are the
    // head's column of row 0, and each copy adds its own row)
    const int64_t kv_off = PAGED ? (int64_t)g * D * 2 : (ks + k_lo) * row_stride + (int64_t)g * D * 2;
    const char *kbase = reinterpret_cast<const char *>(p.k) + kv_off;
    const char *vbase = reinterpret_cast<const char *>(p.v) + kv_off;
    const uint32_t ring = (uint32_t)(uintptr_t)smem;

    // ---- DMA role: the first NW/2 waves copy the K half of every chunk, the
    // others the V half; wave w copies parts part0 .. part0 + PW - 1 of its
    // half.  Lane offsets are chunk-relative source bytes; for the last chunk
    // the keys are clamped to the slice, so every source row is a valid row of
    // the request.
    const bool dv = wave >= NW / 2;
    const int part0 = (wave % (NW / 2)) * PW;
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

    // ---- token-table path.  A copy needs the cache row of each of its keys.
    // In the loop the rows come by scalar loads (their own counter, apart
    // from the copies' vector-memory counter, so the copy waits are the same
    // as without a table): the rows of the next period's chunks are loaded
    // right after this period's chunks are copied, into the same registers,
    // and have a whole period to arrive.  A copy covers groups of 4 cache rows
    // whose keys are consecutive (also in the K order key_of_slot), so a lane
    // picks its row from the 4 values of its group.  Keys past the slice end
    // are clamped to its last key, as in the contiguous path.
    constexpr int RPD = Gm::kRowsPerDma;
    constexpr int G4 = RPD / 4;  // groups of 4 rows per copy
    typedef __attribute__((address_space(4))) const int32_t const_i32_t;
    const_i32_t *tab =
        reinterpret_cast<const_i32_t *>((uintptr_t)(PAGED ? p.table + (int64_t)b * p.tstride + k_lo : nullptr));
    // first key of group gi of copy jj of this wave (wave-uniform)
    auto group_key = [&](int jj, int gi) __attribute__((always_inline)) {
        const int row = (part0 + jj) * RPD + 4 * gi;
        return dv ? row : key_of_slot(row);
    };
    uint32_t goff[PW];  // the lane's 16-byte granule within its row (as in dma_off)
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int byte = (part0 + j) * 1024 + lane * 16;
        const int row = byte / Gm::kRowBytes;
        const int pos = (byte % Gm::kRowBytes) >> 4;
        goff[j] = (uint32_t)((pos ^ (dv ? v_swz<D>(row) : k_swz<D>(row))) << 4);
    }
    const int lrow = (lane * 16) / Gm::kRowBytes;  // the lane's row within a copy (0 .. RPD-1)
    bool slot_bad = false;  // a table entry outside the cache (reported at the end)
    // Copy jj of chunk c into ring stage `stage` from cache row `row`.
    auto copy_row = [&](uint32_t stage, int jj, int32_t row_in) __attribute__((always_inline)) {
        uint32_t row = (uint32_t)row_in;
        if (row >= (uint32_t)p.kvr32) {
            slot_bad = true;
            row = 0;
        }
        const char *a = dbase + (int64_t)row * row_stride + goff[jj];
        dma16_at(a, __builtin_amdgcn_readfirstlane(dlds + stage * kHalf + jj * 1024));
    };
    // The rows of one period's chunks, wave-uniform (scalar registers).
    int32_t srow[PAGED ? BP : 1][PW][G4][4];
    auto load_rows = [&](int cc, int c) __attribute__((always_inline)) {
        const int cap = c == clamp_c ? last_keys - 1 : kChunk - 1;
#pragma unroll
        for (int jj = 0; jj < PW; ++jj)
#pragma unroll
            for (int gi = 0; gi < G4; ++gi)
#pragma unroll
                for (int e = 0; e < 4; ++e) srow[cc][jj][gi][e] = tab[c * kChunk + min(group_key(jj, gi) + e, cap)];
    };
    // (each candidate goes through an empty asm first: the selection is then
    // among plain values, which the compiler cannot turn back into an indexed
    // load from the array, an index that would move the array to scratch)
    auto issue_rows = [&](int cc, int c) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < PW; ++jj) {
            int32_t v = 0;
#pragma unroll
            for (int k = 0; k < 4 * G4; ++k) {
                int32_t x = srow[cc][jj][k >> 2][k & 3];
                asm volatile("" : "+s"(x));
                v = lrow == k ? x : v;
            }
            copy_row((uint32_t)(c % kStages), jj, v);
        }
    };

    // ---- prologue --------------------------------------------------------------
    // (1) the packed ancestor rows of the tile's nodes -> LDS, if the slice
    // reaches the tree tail (4 bytes per lane; offsets clamped into the rows).
    uint64_t *anc_lds = reinterpret_cast<uint64_t *>(smem + Gm::kRingBytes);
    if (k_hi > P) {
        const int nbytes = (node_last - node_first + 1) * p.words * 8;
        const char *src = reinterpret_cast<const char *>(p.anc + ((int64_t)lo + node_first) * p.words);
        const int nblk = (nbytes + 255) / 256;
        for (int blk = wave; blk < nblk; blk += NW) {
            const uint32_t off = (uint32_t)min(blk * 256 + lane * 4, nbytes - 4);
            dma4(src, off, __builtin_amdgcn_readfirstlane(ring + Gm::kRingBytes + blk * 256));
        }
    }
    // (2) this lane's query rows (one per 32-row block) -> registers
    // (asynchronous; waited below).  Rows past the tile repeat a valid one.
    const bool active = row0 + wave * 32 * RB < row_end;  // wave-uniform: the wave has rows
    int r[RB], node[RB], head[RB];
    bool row_ok[RB];
    bf16x8_t qb[RB][KS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        r[rb] = row0 + (wave * RB + rb) * 32 + col;
        row_ok[rb] = r[rb] < row_end;
        node[rb] = row_ok[rb] ? r[rb] / G : node_last;
        head[rb] = g * G + (row_ok[rb] ? r[rb] % G : 0);
        const uint16_t *qrow = p.q + (((int64_t)lo + node[rb]) * p.hq + head[rb]) * D + 8 * half;
#pragma unroll
        for (int k16 = 0; k16 < KS; ++k16)
            asm volatile("global_load_dwordx4 %0, %1, off offset:%2"
                         : "=v"(qb[rb][k16])
                         : "v"(qrow), "n"(32 * k16)
                         : "memory");
    }
    // (2b) RoPE on: the (cos, sin) pairs of the lane's channels i < D/2
    // (channel i is paired with i + D/2: q granule k16 with k16 + KS/2, same
    // lane), 8 pairs per granule.
    const bool rope = p.rope_cs != nullptr;  // uniform
    float4 csv[RB][KS / 2][4];
    if (rope) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float2 *csrow = p.rope_cs + ((int64_t)lo + node[rb]) * (D / 2) + 8 * half;
#pragma unroll
            for (int k16 = 0; k16 < KS / 2; ++k16)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    asm volatile("global_load_dwordx4 %0, %1, off offset:%2"
                                 : "=v"(csv[rb][k16][u])
                                 : "v"(csrow), "n"(128 * k16 + 16 * u)
                                 : "memory");
        }
    }
    // (2c) token table: each lane loads the rows of its copies of chunks
    // 0 .. AH-1 (all of them, chunks past the slice re-reading its last one,
    // so that they are all in flight at once), and the first period's chunks
    // AH .. AH+BP-1 come by scalar loads.
    int32_t prow[PAGED ? AH : 1][PW];
    if constexpr (PAGED) {
        const int32_t *tabv = p.table + (int64_t)b * p.tstride + k_lo;
#pragma unroll
        for (int ch = 0; ch < AH; ++ch) {
            const int chc = min(ch, n - 1);
            const int cap = chc == clamp_c ? last_keys - 1 : kChunk - 1;
#pragma unroll
            for (int jj = 0; jj < PW; ++jj)
                prow[ch][jj] = tabv[chc * kChunk + min(group_key(jj, lrow >> 2) + (lrow & 3), cap)];
        }
#pragma unroll
        for (int cc = 0; cc < BP; ++cc)
            if (AH + cc < n) load_rows(cc, AH + cc);
        // One wait for all of them here (the compiler's, for this use), not
        // one per copy below: a compiler wait between two copies would also
        // wait for the copies already issued, which it does not count.
#pragma unroll
        for (int ch = 0; ch < AH; ++ch)
#pragma unroll
            for (int jj = 0; jj < PW; ++jj) asm volatile("" : "+v"(prow[ch][jj]));
    }
    // (3) the first AH chunks.  While they land, Q is multiplied by
    // c = scale * log2(e) (scores in log2 units; rotated first when RoPE is
    // on) and rounded to bf16 again; after the second wait everything but
    // chunks 2 .. AH-1 has landed (the ancestor rows, Q, chunks 0 and 1).
#pragma unroll
    for (int ch = 0; ch < AH; ++ch) {
        if (ch < n) {
            if constexpr (PAGED) {
#pragma unroll
                for (int jj = 0; jj < PW; ++jj) copy_row((uint32_t)ch, jj, prow[ch][jj]);
            } else {
                issue(ch, ch);
            }
        }
    }
    wait_chunks<PW, AH>(min(n, AH));  // Q, the ancestor rows, the (cos, sin) pairs
    const float c = p.c;
    if (rope) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int k16 = 0; k16 < KS / 2; ++k16) {
                asm volatile("" : "+v"(qb[rb][k16]), "+v"(qb[rb][k16 + KS / 2]));
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const float4 cs4 = csv[rb][k16][e2];  // (cos, sin) of channels 2 e2, 2 e2 + 1
                    const float a0 = (float)qb[rb][k16][2 * e2], a1 = (float)qb[rb][k16][2 * e2 + 1];
                    const float b0 = (float)qb[rb][k16 + KS / 2][2 * e2];
                    const float b1 = (float)qb[rb][k16 + KS / 2][2 * e2 + 1];
                    const f32x2_t x = {(a0 * cs4.x - b0 * cs4.y) * c, (a1 * cs4.z - b1 * cs4.w) * c};
                    const f32x2_t y = {(b0 * cs4.x + a0 * cs4.y) * c, (b1 * cs4.z + a1 * cs4.w) * c};
                    const bf16x2_t xb = __builtin_convertvector(x, bf16x2_t);
                    const bf16x2_t yb = __builtin_convertvector(y, bf16x2_t);
                    qb[rb][k16][2 * e2] = xb[0];
                    qb[rb][k16][2 * e2 + 1] = xb[1];
                    qb[rb][k16 + KS / 2][2 * e2] = yb[0];
                    qb[rb][k16 + KS / 2][2 * e2 + 1] = yb[1];
                }
            }
    } else {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int k16 = 0; k16 < KS; ++k16) {
                asm volatile("" : "+v"(qb[rb][k16]));
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const f32x2_t x = {(float)qb[rb][k16][2 * e2] * c, (float)qb[rb][k16][2 * e2 + 1] * c};
                    const bf16x2_t y = __builtin_convertvector(x, bf16x2_t);
                    qb[rb][k16][2 * e2] = y[0];
                    qb[rb][k16][2 * e2 + 1] = y[1];
                }
            }
    }
    wait_chunks<PW, AH - 2>(min(n, AH) - 2);
    lds_barrier();

    // Top of step j, at every BP-th step: this wave's part of chunk
    // min(j + BP, n - 1) has landed (chunks j + BP + 1 .. j + AH - 1 may still
    // be in flight), then the barrier makes every wave's part visible, then
    // the copies of chunks j + AH .. j + AH + BP - 1 start.  Between barriers
    // the waves drift freely, so the two waves of a SIMD fill each other's
    // gaps.
    // (Token table: this period's chunks are copied with the rows loaded one
    // period earlier, then the next period's rows are loaded.)
    auto step_top = [&](int j) __attribute__((always_inline)) {
        if (j % BP == 0) {
            wait_chunks<PW, AH - 1 - BP>(min(AH - 1 - BP, n - 1 - BP - j));
            lds_barrier();
            if constexpr (PAGED) {
#pragma unroll
                for (int cc = 0; cc < BP; ++cc)
                    if (j + AH + cc < n) issue_rows(cc, j + AH + cc);
#pragma unroll
                for (int cc = 0; cc < BP; ++cc)
                    if (j + AH + BP + cc < n) load_rows(cc, j + AH + BP + cc);
            } else {
#pragma unroll
                for (int c = j + AH; c < j + AH + BP; ++c)
                    if (c < n) issue(c, (uint32_t)(c % kStages));
            }
        }
    };
    if (!active) {
        // A wave without rows only keeps the copy schedule and the barriers.
        for (int j = 0; j < n; ++j) step_top(j);
        if (PAGED && slot_bad) report(p.err, TV_DEVERR_BAD_SLOT, b);
        return;
    }

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
    auto read_k1 = [&](uint32_t base, uint32_t tx, int k16) {
        return *reinterpret_cast<const bf16x8_t *>(smem + (((32u * k16) ^ tx) + base));
    };
    auto read_v1 = [&](uint32_t base, uint32_t tx, int tt, int db) {
        const uint32_t a0 = ((64u * db) ^ tx) + base + (8 * tt) * Gm::kRowBytes;
        const bf16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(smem + a0));
        const bf16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(smem + a0 + 4 * Gm::kRowBytes));
        return bf16x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    };

    f32x16_t oacc[RB][DB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[rb][db][e] = 0.f;
    const f32x16_t zero16 = {};
    // m_run: the reference M in log2 units (-inf until a row sees a key);
    // nb = -M (0 while M is -inf), also held as a splat vector, the starting
    // value of the Q K^T accumulator.
    float m_run[RB], l_run[RB], nb[RB];
    f32x16_t nbv[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
        nb[rb] = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) nbv[rb][e] = 0.f;
    }
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    lds_u64_t *arow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
        arow[rb] = reinterpret_cast<lds_u64_t *>((uint32_t)(uintptr_t)anc_lds +
                                                 (uint32_t)((node[rb] - node_first) * p.words * 8));

    // One score accumulator per 32-row block (S(j), then S(j+1) over it),
    // and two weight sets that alternate between steps: step j takes the
    // softmax of S(j) into W[j & 1] while its products use W[(j+1) & 1] =
    // P(j-1).
    f32x16_t S[RB];
    bf16x8_t W0[RB][2], W1[RB][2];
    // Operand ring: a product's K or V operand is read from LDS kLead
    // operands ahead of its use into slot (operand number) % kSlots, so only
    // a few operands are in flight instead of a whole step's.
    constexpr int kLead = 2;
    constexpr int kSlots = 4;
    static_assert(kLead < kSlots && KS % kSlots == 0 && (2 * DB) % kSlots == 0, "operand ring");
    bf16x8_t opr[kSlots];

    // Mask of chunk j on the scores (a uniform branch before the scheduled
    // block: only chunks that reach the tree tail or the slice end need it).
    auto apply_mask = [&](f32x16_t(&sv)[RB], int j) {
        if (j >= c_mask) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const uint32_t vis = visible16(arow[rb], p.words, k_lo + j * kChunk + 16 * half, P, k_hi);
                if (vis != 0xFFFFu) {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (!((vis >> e) & 1u)) sv[rb][e] = -INFINITY;
                }
            }
        }
    };
    // The weights 2^(s c - m c) at the current reference, rounded to bf16,
    // and their sum (two partial sums halve the dependent chain).
    // The weights 2^(x + shift) of the 16 scores x of one row block, rounded
    // to bf16, and their sum (two partial sums halve the dependent chain).
    auto weights = [&](const f32x16_t &sv, bf16x8_t(&pw)[2], float shift) {
        float l0 = 0.f, l1 = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int j2 = 0; j2 < 4; ++j2) {
                const f32x2_t pf = {__builtin_amdgcn_exp2f(sv[8 * tt + 2 * j2] + shift),
                                    __builtin_amdgcn_exp2f(sv[8 * tt + 2 * j2 + 1] + shift)};
                const bf16x2_t pp = __builtin_convertvector(pf, bf16x2_t);
                if (j2 & 1) l1 = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l1, false);
                else l0 = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l0, false);
                pw[tt][2 * j2] = pp[0];
                pw[tt][2 * j2 + 1] = pp[1];
            }
        }
        return l0 + l1;
    };
    // One step, in two halves of segments that the compiler may not reorder
    // across (sched_barrier); each segment issues the LDS read of the operand
    // kLead places ahead and the RB products (one per row block) that share
    // the current operand.  First half: O += P(j-1) V(j-1) (V^T blocks
    // (tt, db) of chunk j-1), each segment also taking a slice of the
    // softmax of S(j): the weights at the reference in force (speculatively)
    // and the row maxima.  Then the rare raise of a reference (rescale of l
    // and O, the weights again).  Second half: S(j+1) = Q K(j+1)^T (K blocks
    // k16 of chunk j+1), written over S(j), starting from -M.  The step ends
    // with the reads of the first kLead operands of the next PV products,
    // V(j).  Step 0 has no PV products and step n-1 no QK products.
    constexpr int NPVO = 2 * DB;           // PV operands per step
    constexpr int NE = 16 * RB;            // score elements per lane
    constexpr int EPP = (NE + NPVO * RB - 1) / (NPVO * RB);  // elements per PV segment
    auto step = [&](auto pv_, auto qk_, bf16x8_t(&wprev)[RB][2], bf16x8_t(&wcur)[RB][2], int j) {
        constexpr bool PV = decltype(pv_)::value, QK = decltype(qk_)::value;
        step_top(j);
        apply_mask(S, j);
        const uint32_t vprev = vb + (uint32_t)(max(j - 1, 0) % kStages) * kHalf;  // V(j-1), V(0) at step 0
        const uint32_t kcur = kb + (uint32_t)(min(j + 1, n - 1) % kStages) * kHalf;  // K(j+1)
        const uint32_t vcur = vb + (uint32_t)(j % kStages) * kHalf;                // V(j)
        uint32_t vtt = vt, ktt = kt;
        asm volatile("" : "+v"(vtt), "+v"(ktt));
        auto read_op = [&](int o) {
            return o < NPVO ? read_v1(vprev, vtt, o / DB, o % DB) : read_k1(kcur, ktt, o - NPVO);
        };
        float pf[NE];
        float mxp[RB], l0[RB], l1[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            mxp[rb] = -INFINITY;
            l0[rb] = 0.f;
            l1[rb] = 0.f;
        }
        // softmax slice: score elements e0 .. e0 + EPP - 1 (element e is
        // entry e % 16 of row block e / 16)
        auto vec_piece = [&](int e0) {
#pragma unroll
            for (int e = e0; e < e0 + EPP; ++e) {
                if (e < NE) {
                    const int rb = e / 16, el = e % 16;
                    pf[e] = __builtin_amdgcn_exp2f(S[rb][el]);
                    if (el & 1) {
                        mxp[rb] = fmaxf(fmaxf(mxp[rb], S[rb][el - 1]), S[rb][el]);
                        const f32x2_t pr = {pf[e - 1], pf[e]};
                        const bf16x2_t pp = __builtin_convertvector(pr, bf16x2_t);
                        wcur[rb][el >> 3][(el & 7) - 1] = pp[0];
                        wcur[rb][el >> 3][el & 7] = pp[1];
                        if ((el >> 1) & 1) l1[rb] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l1[rb], false);
                        else l0[rb] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l0[rb], false);
                    }
                }
            }
        };
        // first half: PV products with the softmax of S(j) (step 0 has no
        // products: the softmax runs alone, and the QK half's first operands
        // are read here instead)
        if constexpr (PV) {
#pragma unroll
            for (int o = 0; o < NPVO; ++o) {
                opr[(o + kLead) % kSlots] = read_op(o + kLead);  // (o + kLead < NPVO + KS always)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int tt = o / DB, db = o % DB;
                    oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opr[o % kSlots], wprev[rb][tt],
                                                                           oacc[rb][db], 0, 0, 0);
                    vec_piece((o * RB + rb) * EPP);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
#pragma unroll
            for (int o = NPVO; o < NPVO + kLead; ++o) opr[o % kSlots] = read_op(o);
#pragma unroll
            for (int e0 = 0; e0 < NE; e0 += EPP) vec_piece(e0);
        }
        float lsum[RB], mx[RB];
        bool raise = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            lsum[rb] = l0[rb] + l1[rb];
            mx[rb] = halves_max(mxp[rb]);  // relative to the reference in force
            raise |= (mx[rb] > kRescaleLog2) | ((m_run[rb] == -INFINITY) & (mx[rb] > -INFINITY));
            // (the speculative weights are used whatever the branch below
            // does, so they stay interleaved with the products above)
            asm volatile("" : "+v"(wcur[rb][0]), "+v"(wcur[rb][1]), "+v"(lsum[rb]));
        }
        // Rare: the chunk raises a reference (or gives a row its first).
        // Rescale l and O (which now includes P(j-1) V(j-1)) and take the
        // weights again.  A row whose maximum stays within its threshold may
        // be raised too, which changes nothing but rounding.
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float mn = fmaxf(m_run[rb], mx[rb] - nb[rb]);  // new reference
                const float nbn = (mn == -INFINITY) ? 0.f : -mn;       // (a row with no key yet keeps 0)
                const float delta = nbn - nb[rb];
                const float alpha = __builtin_amdgcn_exp2f(m_run[rb] + nbn);  // 0 while m_run is -inf
                l_run[rb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[rb][db][e] *= alpha;
#pragma unroll
                for (int e = 0; e < 16; ++e) nbv[rb][e] = nbn;
                m_run[rb] = mn;
                nb[rb] = nbn;
                lsum[rb] = weights(S[rb], wcur[rb], delta);
            }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) l_run[rb] += lsum[rb];
        // second half: QK products, S(j+1) over S(j) (none at the last step)
        if constexpr (QK) {
#pragma unroll
            for (int o = NPVO; o < NPVO + KS; ++o) {
                if (o + kLead < NPVO + KS) opr[(o + kLead) % kSlots] = read_op(o + kLead);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int k16 = o - NPVO;
                    S[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opr[o % kSlots], qb[rb][k16],
                                                                    k16 ? S[rb] : nbv[rb], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        // the next PV products' first operands: V(j) blocks 0 .. kLead-1
#pragma unroll
        for (int o = 0; o < kLead; ++o) opr[o] = read_v1(vcur, vtt, o / DB, o % DB);
    };

    // Prologue products: S(0) = Q K(0)^T.
    {
        uint32_t ktt = kt, vtt = vt;
        asm volatile("" : "+v"(ktt), "+v"(vtt));
#pragma unroll
        for (int k16 = 0; k16 < KS; ++k16) {
            const bf16x8_t kop = read_k1(kb, ktt, k16);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                S[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qb[rb][k16], k16 ? S[rb] : zero16, 0, 0, 0);
        }
        (void)vtt;
    }
    // Steps alternate the weight sets: even steps take the softmax into W0,
    // odd steps into W1.  Step 0 (no PV products) and step n-1 (no QK
    // products) are peeled off the loop.
    using T_ = std::true_type;
    using F_ = std::false_type;
    if (n == 1) {
        step(F_{}, F_{}, W1, W0, 0);
    } else {
        step(F_{}, T_{}, W1, W0, 0);
        int j = 1;
        for (; j + 2 < n; j += 2) {
            step(T_{}, T_{}, W0, W1, j);      // odd j
            step(T_{}, T_{}, W1, W0, j + 1);  // even j
        }
        if (j + 1 < n) {  // one full step left (odd j)
            step(T_{}, T_{}, W0, W1, j);
            ++j;
        }
        if (j & 1) step(T_{}, F_{}, W0, W1, j);  // j == n - 1
        else step(T_{}, F_{}, W1, W0, j);
    }
    // Last products: O += P(n-1) V(n-1) (V(n-1) blocks 0 .. kLead-1 were read
    // at the end of step n - 1).
    {
        const bool odd = (n - 1) & 1;
        const uint32_t vlast = vb + (uint32_t)((n - 1) % kStages) * kHalf;
        uint32_t vtt = vt;
        asm volatile("" : "+v"(vtt));
#pragma unroll
        for (int o = 0; o < 2 * DB; ++o) {
            if (o + kLead < 2 * DB) opr[(o + kLead) % kSlots] = read_v1(vlast, vtt, (o + kLead) / DB, (o + kLead) % DB);
            const int tt = o / DB, db = o % DB;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opr[o % kSlots], odd ? W1[rb][tt] : W0[rb][tt],
                                                                       oacc[rb][db], 0, 0, 0);
        }
    }

    // ---- epilogue ----------------------------------------------------------------
    if (PAGED && slot_bad) report(p.err, TV_DEVERR_BAD_SLOT, b);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float lr = halves_sum(l_run[rb]);
        if (pc.pslot < 0) {
            if (!row_ok[rb]) continue;
            const float inv = 1.f / lr;
            uint16_t *orow = p.out + (((int64_t)lo + node[rb]) * p.hq + head[rb]) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int d = db * 32 + 8 * i4 + 4 * half;
                    const uint32_t w0 = pack_bf16x2(oacc[rb][db][4 * i4 + 0] * inv, oacc[rb][db][4 * i4 + 1] * inv);
                    const uint32_t w1 = pack_bf16x2(oacc[rb][db][4 * i4 + 2] * inv, oacc[rb][db][4 * i4 + 3] * inv);
                    *reinterpret_cast<uint2 *>(orow + d) = make_uint2(w0, w1);
                }
        } else {
            // Partial of this slice for one 32-row group: O / l rounded to
            // bf16 (a convex combination of V rows, so bf16 keeps its range)
            // plus the fp32 (m, l).  Lane-native layout
            // [slot][row group][DB*4 x 4 bf16][64 lanes].  A row that
            // sees no key of the slice has l = 0 and stores zeros.  The
            // stores are relaxed atomics at agent scope, which write through
            // this XCD's L2: the merge kernel reads them from another XCD
            // anyway, and the end of this kernel then has no dirty partials
            // left to write back (measured: 1.5 us less per call at 240
            // workgroups).
            const int64_t unit = pc.pslot * (NW * RB) + wave * RB + rb;
            uint2 *po = p.ws_o + unit * (DB * 4 * 64) + lane;
            const float inv = lr > 0.f ? 1.f / lr : 0.f;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const uint64_t w =
                        (uint64_t)pack_bf16x2(oacc[rb][db][4 * i4 + 0] * inv, oacc[rb][db][4 * i4 + 1] * inv) |
                        ((uint64_t)pack_bf16x2(oacc[rb][db][4 * i4 + 2] * inv, oacc[rb][db][4 * i4 + 3] * inv)
                         << 32);
                    __hip_atomic_store(reinterpret_cast<uint64_t *>(po + (db * 4 + i4) * 64), w, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            if (half == 0) {
                const uint64_t w = (uint64_t)__float_as_uint(m_run[rb]) | ((uint64_t)__float_as_uint(lr) << 32);
                __hip_atomic_store(reinterpret_cast<uint64_t *>(p.ws_ml + unit * 32 + col), w, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}


// One workgroup per task of the static or planned order (decode_task).
template <int D, int NW, int RB, int AH, bool PAGED>
__global__ void __launch_bounds__(64 * NW, 1) attn_fwd_kernel(KParams p) {
    using Gm = Geo<D, NW, RB>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Gm::kRingBytes + kAncBytes];
    Task tk;
    if (!decode_task(p, blockIdx.x, &tk)) return;
    Piece pc;
    pc.b = tk.b;
    pc.g = tk.g;
    pc.rt = tk.rt;
    pc.k_lo = tk.s * p.keys_per_split;
    pc.k_span = p.keys_per_split;
    pc.pslot = p.splits == 1 ? -1 : ((int64_t)(tk.b * p.hkv + tk.g) * p.row_tiles + tk.rt) * p.splits + tk.s;
    pc.report_bad = tk.g == 0 && tk.rt == 0 && tk.s == 0;
    pc.empty_partial = false;  // (the merge skips the slices past a tile's keys)
    attn_piece<D, NW, RB, AH, PAGED>(p, smem, pc, threadIdx.x);
}

// Balanced order: a fixed grid of kBalWgs workgroups (one per CU), each
// running its own list of pieces one after the other (attn_bal_plan_kernel).
// Between two pieces a barrier lets every wave finish its LDS reads of the
// previous piece before the rings are refilled; no copy is in flight then
// (each wave waits for all of its copies before the last chunk is read).
constexpr int kBalWgs = 256;
template <int D, int NW, int RB, int AH, bool PAGED>
__global__ void __launch_bounds__(64 * NW, 1) attn_fwd_bal_kernel(KParams p) {
    using Gm = Geo<D, NW, RB>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Gm::kRingBytes + kAncBytes];
    const int2 range = p.bal_wg[blockIdx.x];
    // (every entry is checked against the tables' bounds before use)
    if (range.x < 0 || range.y < 0 || range.y > p.bal_slots - range.x) return;
    for (int i = 0; i < range.y; ++i) {
        if (i > 0) __syncthreads();
        const int4 e = p.bal_piece[range.x + i];
        if (e.x < 0 || e.x >= p.batch * p.hkv * p.row_tiles || e.y < 0 || e.z <= e.y || e.w >= p.bal_slots) continue;
        const int q = e.x / p.row_tiles;
        Piece pc;
        pc.rt = e.x - q * p.row_tiles;
        pc.g = q % p.hkv;
        pc.b = q / p.hkv;
        pc.k_lo = e.y * kChunk;
        pc.k_span = (e.z - e.y) * kChunk;
        pc.pslot = e.w;
        pc.report_bad = false;  // (the planner reports invalid requests)
        pc.empty_partial = true;
        // (the thread id made opaque: what the piece derives from it is
        // formed inside each piece, not hoisted out of this loop and kept
        // live through every piece)
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        attn_piece<D, NW, RB, AH, PAGED>(p, smem, pc, tid);
    }
}

// Merge the per-slice partials of one row of one (tile, 32-row group,
// channels): O = sum_s w_s O_s / sum_s w_s l_s with w_s = 2^(m_s - M),
// M = max_s m_s (the slices' references, in log2 units).  One wavefront per (tile, row group, 32-channel block, I4W of
// the 4 float4 slots), four per workgroup; lane layout as the partials (lane
// half h holds channels 32 db + 8 i4 + 4 h .. +3 of row col).  The slices are
// taken in batches whose loads are all issued before any is used, so a batch
// costs one memory round trip; a batch loads only the slices that exist.  With
// few slices (I4W = 4) a wave merges all four slots: four times fewer waves,
// each with four times the loads in flight.
constexpr int kCombineWaves = 4;
template <int D, int I4W>
__global__ void __launch_bounds__(64 * kCombineWaves) attn_combine_kernel(KParams p) {
    constexpr int DB = D / 32;
    constexpr int kGroups = 4 / I4W;                 // waves per (tile, row group, channel block)
    constexpr int kBatch = I4W == 1 ? 16 : 8;        // slices per batch
    // (wave-uniform: the request's sizes then come by scalar loads, which
    // complete independently of the partials' vector loads)
    const int nw = p.rgroups;  // 32-row groups per tile
    int gw;
    if (p.combine_xcd) {
        // the waves of XCD x (workgroup ids x mod 8) take the tiles of KV
        // heads g = x + 8 m, row tile fastest, then m, then the request
        const int per_tile = kGroups * DB * nw;
        const int x = blockIdx.x % kXcds;
        const int wx = (blockIdx.x / kXcds) * kCombineWaves + (threadIdx.x >> 6);
        const int tix = wx / per_tile;
        const int m = (tix / p.row_tiles) % (p.hkv / kXcds);
        const int bx = tix / (p.row_tiles * (p.hkv / kXcds));
        if (bx >= p.batch) return;
        gw = ((bx * p.hkv + x + kXcds * m) * p.row_tiles + tix % p.row_tiles) * per_tile + (wx - tix * per_tile);
    } else {
        gw = blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
    }
    gw = __builtin_amdgcn_readfirstlane(gw);
    const int i4b = (gw % kGroups) * I4W;
    const int db = (gw / kGroups) % DB;
    const int rg = (gw / (kGroups * DB)) % nw;
    const int tile = gw / (kGroups * DB * nw);
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
    // Balanced order: the tile's pieces are the partial slots
    // (first + i) * row_tiles + rt, i < count; a tile of one piece was
    // written whole by its piece.
    int64_t base = (int64_t)tile * p.splits, step = 1;
    int nbal = 0;
    if (p.bal_group) {
        const int2 gi = p.bal_group[tile / p.row_tiles];
        if (gi.y <= 1 || gi.x < 0 || (int64_t)(gi.x + gi.y) * p.row_tiles > p.bal_slots) return;
        base = (int64_t)gi.x * p.row_tiles + rt;
        step = p.row_tiles;
        nbal = gi.y;
    }
    const float2 *ml = p.ws_ml + (base * nw + rg) * 32 + col;
    const uint2 *po = p.ws_o + (base * nw + rg) * (DB * 4 * 64) + (db * 4 + i4b) * 64 + lane;
    const int64_t kMlStride = step * nw * 32;                   // per slice
    const int64_t kOStride = step * nw * DB * 4 * 64;           // per slice
    float2 m_l[kBatch];
    uint2 o[kBatch][I4W];
    // (one request: every tile has nearly all slices, so the early loads are
    // nearly all used; the balanced order knows the tile's piece count from
    // its group record; in a ragged batch in the other orders short requests
    // have few slices, and the loads wait for the sizes instead)
    const int nb0 = p.bal_group ? min(kBatch, nbal) : (p.batch == 1 ? min(kBatch, p.splits) : 0);  // wave-uniform
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
    const int span = tile_span(rows_b, p.tile_rows);
    const int row0 = rt * span;
    const int row_end = min(rows_b, row0 + span);
    if (row0 + rg * 32 >= row_end) return;  // (wave-uniform) no rows in this group
    const int key_end = P + (row_end - 1) / G + 1;
    const int nsplit = p.bal_group ? nbal : min(p.splits, (key_end + p.keys_per_split - 1) / p.keys_per_split);
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
        const float a = __builtin_amdgcn_exp2f(M - mref);  // 0 when M = -inf (references in log2 units)
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
                const float wl = __builtin_amdgcn_exp2f(m_l[u].x - mref) * m_l[u].y;
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
    const int span = tile_span(rows_b, p.tile_rows);
    const int row0 = rt * span;
    if (row0 >= rows_b) return 0;
    const int row_end = min(rows_b, row0 + span);
    const int key_end = rq.P + (row_end - 1) / G + 1;
    const int k_lo = s * p.keys_per_split;
    if (k_lo >= key_end) return 0;
    const int k_hi = min(k_lo + p.keys_per_split, key_end);
    return (k_hi - k_lo + kChunk - 1) / kChunk;
}

// Chunk count of group (s, request sizes rq): its longest tile's.
__device__ __forceinline__ int group_chunks_of(const KParams &p, const Req &rq, int s) {
    int len = 0;
    for (int rt = 0; rt < p.row_tiles; ++rt) len = max(len, tile_chunks(p, rq, s, rt));
    return len;
}

// One workgroup.  Each thread takes groups tid, tid + kPlanThreads, ...; the
// first kPlanCache of them keep their request sizes and lengths in registers
// from the one round of loads at the start (so the second pass below loads
// nothing), and the group (b, g = 0, s = 0) reports a bad request b.
constexpr int kPlanCache = 4;
__global__ void __launch_bounds__(kPlanThreads) attn_plan_kernel(KParams p, int ngroups, int nslots,
                                                                  int32_t *__restrict__ table) {
    __shared__ int cnt[kPlanBins];
    __shared__ int wsum[kPlanThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int R = p.row_tiles;
    Req creq[kPlanCache];
    int clen[kPlanCache];
#pragma unroll
    for (int c = 0; c < kPlanCache; ++c) {
        const int q = tid + c * kPlanThreads;
        clen[c] = 0;
        if (q < ngroups) creq[c] = load_request(p, q / p.splits / p.hkv);
    }
    for (int i = tid; i < kPlanBins; i += kPlanThreads) cnt[i] = 0;
    for (int i = tid; i < nslots; i += kPlanThreads) table[i] = -1;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kPlanCache; ++c) {
        const int q = tid + c * kPlanThreads;
        if (q < ngroups) {
            const int s = q % p.splits, g = (q / p.splits) % p.hkv;
            if (!creq[c].ok) {
                if (s == 0 && g == 0) report(p.err, TV_DEVERR_BAD_REQUEST, q / p.splits / p.hkv);
            } else {
                clen[c] = group_chunks_of(p, creq[c], s);
                if (clen[c] > 0) atomicAdd(&cnt[clen[c]], 1);
            }
        }
    }
    for (int q = tid + kPlanCache * kPlanThreads; q < ngroups; q += kPlanThreads) {
        const int s = q % p.splits, g = (q / p.splits) % p.hkv;
        const Req rq = load_request(p, q / p.splits / p.hkv);
        if (!rq.ok) {
            if (s == 0 && g == 0) report(p.err, TV_DEVERR_BAD_REQUEST, q / p.splits / p.hkv);
            continue;
        }
        const int len = group_chunks_of(p, rq, s);
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
    // Group q of length len > 0 with request sizes rq -> its tiles' slots.
    auto place = [&](int q, int len, const Req &rq) {
        const int k = atomicAdd(&cnt[len], 1);  // rank of the group, longest first
        const int s = q % p.splits;
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
    };
#pragma unroll
    for (int c = 0; c < kPlanCache; ++c) {
        const int q = tid + c * kPlanThreads;
        if (q < ngroups && clen[c] > 0) place(q, clen[c], creq[c]);
    }
    for (int q = tid + kPlanCache * kPlanThreads; q < ngroups; q += kPlanThreads) {
        const Req rq = load_request(p, q / p.splits / p.hkv);
        if (!rq.ok) continue;
        const int len = group_chunks_of(p, rq, q % p.splits);
        if (len > 0) place(q, len, rq);
    }
}


// Balanced plan for batches (TV_ORDER_BALANCED).  The work of a group
// (request b, KV head g) is its R_b row tiles (R_b = ceil(N_b G / tile rows))
// over L_b chunks (the last tile's keys; the others see a few less).  The
// R_b tiles of one key range read the same K/V, so they run together on R_b
// workgroups of one XCD, a "lane" of width R_b.  Groups of equal width form a
// class; laid end to end (requests in order, KV heads within a request), each
// group takes kBalPieceCost positions (its piece's prologue) and then one
// position per chunk.  Class c gets x_c lanes of width c, x_c in proportion to
// its positions W_c, so that every lane has W_c / x_c positions, the same for
// every class, and the lanes fill the kBalWgs workgroups.  Lane i of class c
// takes the chunks whose positions lie in [i W_c / x_c, (i + 1) W_c / x_c):
// one piece per group with such chunks, usually one or two.  A group cut into
// several pieces has partials (C pieces in partial slots F .. F + C - 1, each
// times R_max plus the row tile); a group left whole writes its output
// directly.  Piece numbers F = (pieces before class c) + i + rank of the group
// in its class are unique: along a class both the lane and the group rank
// only grow, one of them at every cut.  A lane holds at least one position,
// so the lanes between a group's first and last chunk all hold some of its
// chunks.  Workgroup ids: lane l of the kBalWgs is id (l / 32) + 8 (l % 32)
// (32 consecutive lanes per XCD, so a lane's tiles share that XCD's L2).
// One thread per request (batch <= kBalThreads), then one per lane.
constexpr int kBalThreads = 1024;
constexpr int kBalMaxWidth = 8;  // row tiles per group the balanced plan takes
constexpr int kBalMaxChunks = 1 << 22;  // positions of all groups together (32-bit plan arithmetic)
// Each group's range opens with this many positions that hold no chunk: the
// cost of a piece's prologue (about 5 us, four chunks of a full tile), so a
// lane that starts a second piece takes that many fewer chunks.
constexpr int kBalPieceCost = 4;
constexpr int kBalWaves = kBalThreads / 64;

__device__ __forceinline__ int bal_wg_of_lane(int l) { return (l >> 5) + 8 * (l & 31); }

// n / d for 0 <= n < 2^31, d > 0 and a quotient of at most 2^22, from the
// hardware reciprocal of d (within one ulp, so the estimate is off by at most
// one) and one correction each way.
__device__ __forceinline__ int bal_div(int n, int d, float inv_d) {
    int q = (int)((float)n * inv_d);
    if ((q + 1) * d <= n) ++q;
    else if (q * d > n) --q;
    return q;
}

// Lane of class position x (0 <= x < W): the largest i with i W / lanes <= x.
// (W <= kBalMaxChunks and lanes <= kBalWgs: every product fits 31 bits.)
__device__ __forceinline__ int bal_lane_of(int x, int W, float inv_W, int lanes) {
    return bal_div((x + 1) * lanes - 1, W, inv_W);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within each row of
// 16 lanes, then the row totals broadcast to the rows after them (DPP moves,
// no LDS round trip).
__device__ __forceinline__ int bal_wave_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false); // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false); // row_bcast:31 -> rows 2, 3
    return x;
}

__global__ void __launch_bounds__(kBalThreads) attn_bal_plan_kernel(KParams p, int2 *__restrict__ wg,
                                                                     int4 *__restrict__ piece,
                                                                     int2 *__restrict__ grp) {
    constexpr int NC = kBalMaxWidth + 1;  // classes 1 .. kBalMaxWidth (0: no work)
    __shared__ int s_cls[kBalThreads], s_len[kBalThreads];
    __shared__ int s_rank[kBalThreads], s_off[kBalThreads];  // by request: rank and first chunk in its class
    __shared__ int s_plen[kBalThreads], s_porder[kBalThreads], s_first[kBalThreads];  // by class position
    __shared__ int s_wcnt[kBalWaves][NC];
    __shared__ int s_wsum[kBalWaves][NC];
    __shared__ int s_cnt[NC], s_W[NC], s_x[NC], s_cstart[NC], s_sbase[NC], s_lane0[NC], s_pbase[NC];
    __shared__ int s_nlanes;
    __shared__ int s_wtot[kBalWaves];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int R = p.row_tiles, hkv = p.hkv, G = p.hq / p.hkv;

    // (1) each request's class (row tiles) and length (chunks of its last
    // tile); within the wave, the requests of its class before it (ballot)
    // and their chunks (prefix sum)
    const int b = tid;
    int cls = 0, len = 0;
    if (b < p.batch) {
        const Req rq = load_request(p, b);
        if (!rq.ok) {
            report(p.err, TV_DEVERR_BAD_REQUEST, b);
        } else if (rq.n > 0) {
            cls = (rq.n * G + p.tile_rows - 1) / p.tile_rows;
            len = (rq.P + rq.n + kChunk - 1) / kChunk;
        }
    }
    const int span = cls > 0 ? len + kBalPieceCost : 0;  // positions of each of its groups
    for (int i = tid; i < kBalWgs; i += kBalThreads) wg[i] = make_int2(0, 0);
    const uint64_t below = (1ull << lane) - 1ull;
    int rank_b = 0, off_b = 0;
#pragma unroll
    for (int c = 1; c < NC; ++c) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(cls == c);
        int incl = 0;
        if (m != 0) {  // (wave-uniform)
            const int xv = cls == c ? span : 0;
            incl = bal_wave_scan(xv);
            if (cls == c) {
                rank_b = __builtin_popcountll(m & below);
                off_b = incl - xv;
            }
        }
        if (lane == 63) {
            s_wcnt[wv][c] = __builtin_popcountll(m);
            s_wsum[wv][c] = incl;
        }
    }
    __syncthreads();
    // (2) across waves: the class totals, and each request's rank and first
    // chunk in its class
    if (tid > 0 && tid < NC) {
        int cnt = 0, sum = 0;
#pragma unroll
        for (int w = 0; w < kBalWaves; ++w) {
            cnt += s_wcnt[w][tid];
            sum += s_wsum[w][tid];
        }
        s_cnt[tid] = cnt;
        s_W[tid] = sum * hkv;  // positions of the class: every KV head of each request
    }
    if (cls > 0) {
#pragma unroll
        for (int w = 0; w < kBalWaves - 1; ++w)
            if (w < wv) {
                rank_b += s_wcnt[w][cls];
                off_b += s_wsum[w][cls];
            }
    }
    s_cls[tid] = cls;
    s_len[tid] = len;
    s_rank[tid] = rank_b;
    s_off[tid] = off_b * hkv;  // the request's groups start here in its class
    __syncthreads();
    // (3) wave 0: lanes per class (the floor of each class's share, at least
    // one, then one more for each class whose remainder is at least a half
    // while lanes are left), laid out widest class first.  Meanwhile the
    // requests take their positions in class order.
    if (wv == 0) {
        int W[NC], x[NC];
        float frac[NC];
        int wtot = 0, used = 0;
#pragma unroll
        for (int c = 1; c < NC; ++c) {
            W[c] = s_W[c];
            wtot += W[c] * c;
        }
        const float share = (float)kBalWgs / (float)max(wtot, 1);
#pragma unroll
        for (int c = 1; c < NC; ++c) {
            x[c] = 0;
            frac[c] = 0.f;
            if (W[c] > 0) {
                const float y = (float)W[c] * share;
                int xi = (int)y;
                frac[c] = y - (float)xi;
                xi = max(1, min(xi, W[c]));
                x[c] = xi;
                used += xi * c;
            }
        }
        // (the floor of one lane per class may overshoot: 8 classes of
        // widths 1 .. 8 need 36 workgroups, so this ends)
        while (used > kBalWgs) {
            int best = 0, bx = 0;
#pragma unroll
            for (int c = 1; c < NC; ++c)
                if (x[c] > 1 && x[c] * c > bx) {
                    best = c;
                    bx = x[c] * c;
                }
#pragma unroll
            for (int c = 1; c < NC; ++c)
                if (c == best) --x[c];
            used -= best;
        }
#pragma unroll
        for (int c = NC - 1; c >= 1; --c)
            if (frac[c] >= 0.5f && c <= kBalWgs - used && x[c] > 0 && x[c] < W[c]) {
                ++x[c];
                used += c;
            }
        if (lane == 0) {
            int l0 = 0, sb = 0, pb = 0;
#pragma unroll
            for (int c = NC - 1; c >= 1; --c) {
                s_x[c] = x[c];
                s_lane0[c] = l0;
                s_sbase[c] = sb;
                s_pbase[c] = pb;
                l0 += x[c] * c;
                sb += x[c];
                pb += x[c] + s_cnt[c] * hkv;
            }
            s_nlanes = sb;
        }
    }
    if (cls > 0) {
        int cst = 0;
#pragma unroll
        for (int c = 1; c < NC; ++c)
            if (c < cls) cst += s_cnt[c];
        s_porder[cst + rank_b] = b;
        s_plen[cst + rank_b] = len;
        s_first[cst + rank_b] = off_b * hkv;
    }
    if (tid > 0 && tid < NC) {
        int cst = 0;
#pragma unroll
        for (int c = 1; c < NC; ++c)
            if (c < tid) cst += s_cnt[c];
        s_cstart[tid] = cst;
    }
    __syncthreads();
    // (4) each group's pieces, for the merge: one thread per group
    for (int q = tid; q < p.batch * hkv; q += kBalThreads) {
        const int rb = q / hkv, g = q - rb * hkv;
        const int c = s_cls[rb];
        int2 gi = make_int2(0, 0);
        if (c > 0) {
            const int Wc = s_W[c], xc = s_x[c];
            const int lb = s_len[rb];
            const int o = s_off[rb] + g * (lb + kBalPieceCost) + kBalPieceCost;  // the group's first chunk
            const float inv = __builtin_amdgcn_rcpf((float)Wc);
            const int i0 = bal_lane_of(o, Wc, inv, xc);
            const int i1 = bal_lane_of(o + lb - 1, Wc, inv, xc);
            gi = make_int2(s_pbase[c] + i0 + s_rank[rb] * hkv + g, i1 - i0 + 1);
        }
        grp[q] = gi;
    }
    // (5) one thread per lane: its pieces, counted, then written after a scan
    // of the counts (times the lane's width) gives each lane its entries
    const int nl = s_nlanes;
    int c = 0, i = 0, count = 0, pos0 = 0, A = 0, E = 0, Wc = 1, xc = 1, cs0 = 0, ncls = 0, pb0 = 0, l00 = 0;
    if (tid < nl) {
#pragma unroll
        for (int cc = 1; cc < NC; ++cc) {
            const int xcc = s_x[cc], sb = s_sbase[cc];
            if (xcc > 0 && tid >= sb && tid < sb + xcc) c = cc;
        }
        Wc = s_W[c];
        xc = s_x[c];
        i = tid - s_sbase[c];
        cs0 = s_cstart[c];
        pb0 = s_pbase[c];
        l00 = s_lane0[c];
        ncls = s_cnt[c];
        const float inv_x = __builtin_amdgcn_rcpf((float)xc);
        A = bal_div(i * Wc, xc, inv_x);
        E = bal_div((i + 1) * Wc, xc, inv_x);
        // the request holding chunk A: the last position whose first chunk <= A
        int lo = cs0, hi = cs0 + ncls - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_first[mid] <= A) lo = mid;
            else hi = mid - 1;
        }
        pos0 = lo;
        // count the groups [A, E) meets
        int pos = pos0, xx = A;
        while (xx < E) {
            const int lb = s_plen[pos] + kBalPieceCost;
            const int gstart = s_first[pos];
            const int g = bal_div(xx - gstart, lb, __builtin_amdgcn_rcpf((float)lb));
            const int o = gstart + g * lb;
            const int gend = o + lb;
            const int xe = min(E, gend);
            // chunks whose position lies in [xx, xe)
            count += max(xx - o - kBalPieceCost, 0) < xe - o - kBalPieceCost;
            xx = xe;
            if (g + 1 == hkv && xx == gend) ++pos;
        }
    }
    // entries of the lanes before this one: a scan of count * width
    const int v = tid < nl ? count * c : 0;
    const int incl = bal_wave_scan(v);
    if (lane == 63) s_wtot[wv] = incl;
    __syncthreads();
    if (tid < nl) {
        int ebase = incl - v;
        for (int w = 0; w < wv; ++w) ebase += s_wtot[w];
        for (int rt = 0; rt < c; ++rt) wg[bal_wg_of_lane(l00 + i * c + rt)] = make_int2(ebase + rt * count, count);
        const float inv_W = __builtin_amdgcn_rcpf((float)Wc);
        int pos = pos0, j = 0, xx = A;
        while (xx < E) {
            const int len_g = s_plen[pos];
            const int lb = len_g + kBalPieceCost;
            const int gstart = s_first[pos];
            const int g = bal_div(xx - gstart, lb, __builtin_amdgcn_rcpf((float)lb));
            const int o = gstart + g * lb;  // the group's positions: kBalPieceCost, then its chunks
            const int gend = o + lb;
            const int xe = min(E, gend);
            const int c0 = max(xx - o - kBalPieceCost, 0), c1 = xe - o - kBalPieceCost;
            if (c0 < c1) {
                const int i0 = bal_lane_of(o + kBalPieceCost, Wc, inv_W, xc);
                const int i1 = bal_lane_of(gend - 1, Wc, inv_W, xc);
                // the group's rank in its class: requests before it times hkv, plus g
                const int pi = pb0 + i + (pos - cs0) * hkv + g;
                const int q = s_porder[pos] * hkv + g;
                for (int rt = 0; rt < c; ++rt)
                    piece[ebase + rt * count + j] = make_int4(q * R + rt, c0, c1, i1 > i0 ? pi * R + rt : -1);
                ++j;
            }
            xx = xe;
            if (g + 1 == hkv && xx == gend) ++pos;
        }
    }
}

}  // namespace

MfmaPlan plan_attn_mfma(int batch, int total_nodes, int max_nodes, int max_prefix, int hq, int hkv,
                        int head_dim, tv_dtype dtype, const tv_attn_plan_override *ov) {
    (void)total_nodes;
    MfmaPlan plan;
    const int G = hkv > 0 ? hq / hkv : 0;
    // Every bf16 call: a tree of fewer than 32 rows per KV head fills part of
    // one 32-row block (the rows past it repeat a valid row and are not
    // stored), and still streams each K/V chunk once per KV head instead of
    // once per (node, head) as the vector kernel does (one node, GQA 4,
    // prefix 8192: 24 us against 2.9 ms).
    if (dtype != TV_BF16 || (head_dim != 64 && head_dim != 128) || batch <= 0 || max_nodes * G < 1)
        return plan;
    plan.use = true;
    // Each wave owns one 32-row block.  8 waves (256-row tiles, two waves
    // per SIMD) let the waves of a SIMD fill each other's gaps; 4 waves
    // (128-row tiles) halve the rows per tile, so a single request needs
    // half the key-axis slices to fill the chip, and writes half the split
    // partials.  Measured (us per call, cold cache): a single request with at
    // most 512 rows per KV head is faster with 4 (c3 28.4 against 30.5, c2
    // 17.3 against 21.4), larger ones and batches with 8 (c4 53.0 against
    // 65.7, c5 89.6 against 111).
    const bool small = batch == 1 && (long)max_nodes * G <= 512;
    plan.waves = (ov && ov->waves) ? ov->waves : (small ? 4 : 8);
    plan.row_blocks = 1;
    plan.rows_per_tile = 32 * plan.waves * plan.row_blocks;
    plan.row_tiles = (max_nodes * G + plan.rows_per_tile - 1) / plan.rows_per_tile;
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
    // Batches: the balanced order (equal shares of the key axis per
    // workgroup, see attn_bal_plan_kernel) unless the override fixes the
    // slices or another order, or the batch is beyond its planner.
    const bool bal_fits = batch <= kBalThreads && plan.row_tiles <= kBalMaxWidth &&
                          (long)batch * hkv * (chunks + kBalPieceCost) <= kBalMaxChunks &&
                          ((long)kBalWgs + (long)batch * hkv) * plan.row_tiles <= INT32_MAX;
    if (batch > 1 && bal_fits &&
        (order == TV_ORDER_BALANCED || (order == TV_ORDER_AUTO && !(ov && ov->splits > 0)))) {
        plan.balanced = true;
        plan.splits = 0;
        plan.keys_per_split = 0;
        const size_t slots = ((size_t)kBalWgs + (size_t)batch * hkv) * plan.row_tiles;
        const size_t rows = slots * plan.rows_per_tile;
        auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
        size_t off = up(rows * head_dim * sizeof(uint16_t));  // partial O
        off = up(off + rows * sizeof(float2));                 // partial (m, l)
        plan.bal_wg_off = off;
        off = up(off + (size_t)kBalWgs * sizeof(int2));
        plan.bal_piece_off = off;
        off = up(off + slots * sizeof(int4));
        plan.bal_group_off = off;
        plan.ws_bytes = off + (size_t)batch * hkv * sizeof(int2);
        return plan;
    }
    const bool can_plan = batch > 1 && order != TV_ORDER_STATIC;
    const long target = batch == 1 ? 256 : (can_plan ? 1024 : 640);
    int splits = (int)((target + base_tasks - 1) / base_tasks);
    // A slice covers at least kMinSliceChunks chunks: below that its split
    // partial (256 B per row) costs more than the keys it streams save
    // (c2, 1088 keys: 7 slices 17.3 us, 12 slices 18.3 us, 17 slices 21.4 us).
    splits = max(1, min(splits, chunks / kMinSliceChunks));
    if (ov && ov->splits > 0) splits = ov->splits;
    if (splits < 1) splits = 1;
    if (splits > chunks) splits = chunks;
    const int cps = (chunks + splits - 1) / splits;  // chunks per split
    plan.keys_per_split = cps * kChunk;
    plan.splits = (chunks + cps - 1) / cps;
    if (plan.splits > 1) {
        const size_t rows = (size_t)base_tasks * plan.splits * plan.rows_per_tile;
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
    if (plan.balanced) return kAhead;
    return plan.keys_per_split / kChunk <= kShortSlice ? kAheadShort : kAhead;
}

namespace {
template <int D, int NW, int RB, bool PAGED>
void launch_fwd_t(const KParams &p, const MfmaPlan &plan, long grid, hipStream_t stream) {
    if (attn_mfma_lookahead(plan) == kAheadShort)
        hipLaunchKernelGGL((attn_fwd_kernel<D, NW, RB, kAheadShort, PAGED>), dim3(grid), dim3(64 * NW), 0, stream, p);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<D, NW, RB, kAhead, PAGED>), dim3(grid), dim3(64 * NW), 0, stream, p);
}
template <int D, int NW, int RB>
void launch_fwd(const KParams &p, const MfmaPlan &plan, long grid, hipStream_t stream) {
    if (plan.balanced) {
        if (p.table)
            hipLaunchKernelGGL((attn_fwd_bal_kernel<D, NW, RB, kAhead, true>), dim3(kBalWgs), dim3(64 * NW), 0,
                               stream, p);
        else
            hipLaunchKernelGGL((attn_fwd_bal_kernel<D, NW, RB, kAhead, false>), dim3(kBalWgs), dim3(64 * NW), 0,
                               stream, p);
        return;
    }
    if (p.table) launch_fwd_t<D, NW, RB, true>(p, plan, grid, stream);
    else launch_fwd_t<D, NW, RB, false>(p, plan, grid, stream);
}
}  // namespace

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
    p.rgroups = plan.rows_per_tile / 32;
    p.tile_rows = plan.rows_per_tile;
    p.row_tiles = plan.row_tiles;
    p.splits = plan.splits;
    p.keys_per_split = plan.keys_per_split;
    p.c = a.scale * kLog2e;
    p.out = (uint16_t *)a.out;
    p.err = a.err;
    p.table = a.table;
    p.tstride = a.table_stride;
    p.kvr32 = (int)(a.kv_rows < INT32_MAX ? a.kv_rows : INT32_MAX);
    p.rope_cs = a.rope_cs;
    p.ws_o = nullptr;
    p.ws_ml = nullptr;
    p.task_table = nullptr;
    p.bal_wg = nullptr;
    p.bal_piece = nullptr;
    p.bal_group = nullptr;
    p.bal_slots = 0;
    p.combine_xcd = (!plan.balanced && !plan.table && a.hkv % kXcds == 0) ? 1 : 0;
    if (plan.balanced) {
        const size_t rows = ((size_t)kBalWgs + (size_t)a.batch * a.hkv) * plan.row_tiles * plan.rows_per_tile;
        const size_t off = (rows * a.head_dim * sizeof(uint16_t) + 255) & ~(size_t)255;
        char *ws = (char *)workspace;
        p.ws_o = (uint2 *)ws;
        p.ws_ml = (float2 *)(ws + off);
        int2 *wg = (int2 *)(ws + plan.bal_wg_off);
        int4 *piece = (int4 *)(ws + plan.bal_piece_off);
        int2 *grp = (int2 *)(ws + plan.bal_group_off);
        p.bal_slots = (int)(((size_t)kBalWgs + (size_t)a.batch * a.hkv) * plan.row_tiles);
        hipLaunchKernelGGL(attn_bal_plan_kernel, dim3(1), dim3(kBalThreads), 0, stream, p, wg, piece, grp);
        p.bal_wg = wg;
        p.bal_piece = piece;
        p.bal_group = grp;
    } else if (plan.splits > 1) {
        const size_t rows = (size_t)a.batch * a.hkv * plan.row_tiles * plan.splits * plan.rows_per_tile;
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
    // (the balanced order cuts a group into a few pieces)
    const bool wide = plan.balanced || plan.splits <= 8;
    const bool merge = plan.balanced || plan.splits > 1;
    const long cwaves = tiles * (plan.rows_per_tile / 32) * (a.head_dim / 32) * (wide ? 1 : 4);
    // XCD-aligned merge: each XCD's waves (tiles / 8 of them) in whole workgroups
    const long cblocks = p.combine_xcd
                             ? kXcds * ((cwaves / kXcds + kCombineWaves - 1) / kCombineWaves)
                             : (cwaves + kCombineWaves - 1) / kCombineWaves;
    if (a.head_dim == 128) {
        if (plan.waves == 8) launch_fwd<128, 8, 1>(p, plan, grid, stream);
        else launch_fwd<128, 4, 1>(p, plan, grid, stream);
        if (merge && wide)
            hipLaunchKernelGGL((attn_combine_kernel<128, 4>), dim3(cblocks), dim3(64 * kCombineWaves), 0, stream, p);
        else if (merge)
            hipLaunchKernelGGL((attn_combine_kernel<128, 1>), dim3(cblocks), dim3(64 * kCombineWaves), 0, stream, p);
    } else {
        if (plan.waves == 8) launch_fwd<64, 8, 1>(p, plan, grid, stream);
        else launch_fwd<64, 4, 1>(p, plan, grid, stream);
        if (merge && wide)
            hipLaunchKernelGGL((attn_combine_kernel<64, 4>), dim3(cblocks), dim3(64 * kCombineWaves), 0, stream, p);
        else if (merge)
            hipLaunchKernelGGL((attn_combine_kernel<64, 1>), dim3(cblocks), dim3(64 * kCombineWaves), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace tv
