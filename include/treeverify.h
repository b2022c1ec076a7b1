/*
 * treeverify.h -- C ABI of libtreeverify, the MI355X (gfx950) tree-verification
 * pass of tree-structured speculative decoding.
 *
 * Pages cited:
 *   [TSD] "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
 *         Tree Attention Accelerate LLM Serving" (llms.blog).
 *   [DT]  "DominoTree: Conditional Tree-Structured Drafting with Domino for
 *         Speculative Decoding" (arXiv 2607.08642).
 *   [DAR] "DARTree: Speculative Diffusion Decoding with Autoregressive Draft
 *         Trees" (gist.science), Technical Summary.
 *
 * A batch holds B requests.  Request b owns:
 *   - draft-tree nodes cu_nodes[b] .. cu_nodes[b+1]-1 of every per-node array
 *     (T = cu_nodes[B] nodes in total; N_b = cu_nodes[b+1] - cu_nodes[b]);
 *   - cache rows kv_start[b] .. kv_start[b] + P_b + N_b - 1 of the K and V
 *     caches: first its prefix (P_b = prefix_len[b] cached tokens), then its
 *     tree node j at row kv_start[b] + P_b + j (tree K/V are appended after the
 *     prefix, [TSD] "KV Cache Rollback").
 * parent[] holds request-local indices: parent[i] < i, or -1 when node i hangs
 * directly under the implicit root, the last verified token ([TSD] "Tree
 * Representation of Speculative Candidates"; parents precede children as in
 * [DT] Appendix B, "Frontier ledger and selection").  A tree whose own root is
 * a node (a bonus token verified in the same pass) is node 0 with parent -1.
 *
 * Conventions for every call:
 *   - All array pointers are caller-owned DEVICE memory on the current HIP
 *     device, contiguous, in the layouts stated.  The library allocates
 *     nothing and keeps no state; calls are thread-safe across streams.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns; nothing synchronises with the host.
 *   - Sizes the host knows (batch, totals, maxima) are passed by value so the
 *     launch needs no device-to-host copy.  Arguments are checked on the host
 *     BEFORE anything is enqueued; a non-zero tv_status means nothing was
 *     enqueued and no output was touched.
 *   - Device-side checks (values held in device arrays) report through the
 *     optional int32 `err` word: 0 = no error, else (code << 24) | index with
 *     the TV_DEVERR_* codes below; when several errors occur the word ends up
 *     holding the largest encoded value (an atomic max), so the result does
 *     not depend on thread timing.  The caller zeroes it beforehand.  A
 *     request that fails a device-side check gets unspecified outputs, but
 *     every memory access stays inside the buffers the sizes describe.
 *   - Element types: tv_dtype selects fp32 or bf16 (bf16 = the upper 16 bits
 *     of an IEEE float32, round-to-nearest-even on output).  Attention
 *     accumulates in fp32 for both.
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TV_OK = 0,
    TV_ERR_NULL = 1,      /* a required pointer is NULL                              */
    TV_ERR_SHAPE = 2,     /* inconsistent or negative sizes (e.g. hq % hkv != 0)      */
    TV_ERR_DTYPE = 3,     /* unsupported dtype / head_dim                             */
    TV_ERR_LIMIT = 4,     /* a size above a library limit (TV_MAX_*)                  */
    TV_ERR_WORKSPACE = 5, /* workspace smaller than the call's *_workspace_size()      */
    TV_ERR_LAUNCH = 6,    /* the HIP runtime refused a launch                         */
    TV_ERR_ALIGN = 7,     /* a pointer breaks the stated alignment                    */
    TV_ERR_SCRATCH = 8    /* the call needs more than the static scratch buffer holds */
} tv_status;

typedef enum { TV_F32 = 0, TV_BF16 = 1 } tv_dtype;

#define TV_MAX_NODES 1024          /* nodes per request                   */
#define TV_MAX_DEPTH 64            /* levels per tree / accepted tokens   */
#define TV_MAX_TOTAL_NODES 16777215 /* nodes per batch (24-bit error index) */
#define TV_MAX_LEDGER 8192         /* ledger slots (depths x lanes) per request */
#define TV_MAX_VOCAB 16777216      /* logits per row                              */
#define TV_GDN_HEAD_DIM 128        /* Gated-DeltaNet q/k and v channels per head   */
#define TV_GDN_MAX_NODES 256       /* nodes per request in tree_gdn_verify         */
#define TV_GDN_MAX_TABLE 4096      /* N_b x max_depth per request in tree_gdn_verify */

/* device error codes (the top byte of the err word) */
#define TV_DEVERR_BAD_PARENT 1  /* parent[v] not in [-1, v); index = global node v       */
#define TV_DEVERR_TOO_DEEP 2    /* level(i) > max_depth; index = global node i           */
#define TV_DEVERR_BAD_REQUEST 3 /* request sizes disagree with the host sizes; index = b */
#define TV_DEVERR_BAD_PATH 4    /* accepted path entry out of range; index = b           */
#define TV_DEVERR_BAD_LEDGER 5  /* chosen slot whose parent is unusable; index = b       */
#define TV_DEVERR_LIMIT 6       /* a request above a per-request limit; index = b        */
#define TV_DEVERR_BAD_SLOT 7    /* token-table entry outside [0, kv_rows); index = b     */
#define TV_DEVERR_BAD_TOKEN 8   /* draft token >= vocab; index = global node             */

/* Human-readable name of a tv_status value (static string). */
const char *tv_status_string(int status);

/* Version of this ABI; bumped on any signature change. */
int tv_abi_version(void);

/*
 * tree_mask_build -- packed ancestor mask, levels and position ids.
 *
 * Defines: [TSD] "The Tree Attention Mechanism", part 2 "2D Causal Tree Mask"
 * (node i may attend to node j iff j is i or an ancestor of i) and part 3
 * "Tree Positional IDs" (a node's position is the root's position plus its
 * depth).  With the root at position P_b - 1 (the last cached token, 0-based),
 * pos[i] = P_b + level[i] - 1, where level[i] counts the nodes on the
 * root->i path (1 for a root child); a chain gets P_b, P_b+1, ..., the
 * ordinary autoregressive positions.
 *
 * In:  parent [T] int32, cu_nodes [B+1] int32, prefix_len [B] int32.
 *      batch = B >= 0; total_nodes = T (the length of the per-node arrays);
 *      max_nodes >= every N_b, 1 <= max_nodes <= TV_MAX_NODES;
 *      1 <= max_depth <= TV_MAX_DEPTH.
 * Out: anc_bits [T, W] uint64 with W = ceil(max_nodes / 64): bit (j & 63) of
 *      word (j >> 6) of row t is set iff request-local node j is t's node or
 *      one of its ancestors (LSB first; no bit at or beyond N_b);
 *      level [T] int32; pos_ids [T] int32.  8-byte aligned anc_bits.
 * err: BAD_PARENT, TOO_DEEP (the node's walk meets them in that order, the
 *      depth check first at each step), BAD_REQUEST (cu_nodes not
 *      non-decreasing within [0, T], N_b > max_nodes, or P_b < 0).
 *      A node with an error gets zero bits, level 0 and pos 0.
 */
tv_status tree_mask_build(const int32_t *parent, const int32_t *cu_nodes, const int32_t *prefix_len,
                          int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_depth,
                          uint64_t *anc_bits, int32_t *level, int32_t *pos_ids, int32_t *err,
                          void *stream);

/*
 * tree_attn_verify_workspace_size -- bytes of device workspace the call below
 * needs for these host sizes (0 when it needs none).  Pure host arithmetic.
 */
size_t tree_attn_verify_workspace_size(int32_t batch, int32_t total_nodes, int32_t max_nodes,
                                       int32_t max_prefix, int32_t hq, int32_t hkv, int32_t head_dim,
                                       tv_dtype dtype);

/*
 * tree_attn_verify -- attention of every tree node over its request's prefix
 * and its own ancestors-or-self.
 *
 * Defines: [TSD] "The Tree Attention Mechanism": the flattened tree is
 * processed in one pass next to the prefix KV cache (part 1 "Tree
 * Flattening"); every node sees the shared prompt history and the nodes on its
 * own branch, never a sibling branch (part 2 "2D Causal Tree Mask"); [DT]
 * section 2.4 calls this verification with an ancestor-only mask.  For node i
 * of request b and query head h, with KV head g = h / (hq / hkv):
 *   out[i,h] = sum_t softmax_t(scale * q[i,h] . k[t,g]) v[t,g]
 *   over t in {kv_start[b] + 0 .. P_b-1} U {kv_start[b] + P_b + j : j in anc(i)}.
 * Q and K arrive with positions already applied (pos_ids above feed the
 * caller's RoPE, or tree_attn_verify_ex applies it).
 *
 * In:  q [T, hq, head_dim]; k_cache, v_cache [kv_rows, hkv, head_dim]
 *      (dtype elements, 16-byte aligned); cu_nodes, kv_start, prefix_len
 *      as above; anc_bits from tree_mask_build with the same max_nodes.
 *      max_prefix >= every P_b; kv_rows = rows of each cache.
 *      head_dim in {64, 128}; hq % hkv == 0; scale > 0 (usually 1/sqrt(d)).
 * Out: out [T, hq, head_dim] in dtype (16-byte aligned).
 * workspace: at least tree_attn_verify_workspace_size(...) bytes, 256-byte
 *      aligned (may be NULL when that size is 0); contents on entry do not
 *      matter and are scratch afterwards.  Calls sharing one workspace must
 *      be ordered on one stream.
 * err: BAD_REQUEST for a request whose N_b > max_nodes, P_b > max_prefix,
 *      P_b < 0, or rows beyond kv_rows; its output rows are not written.
 */
tv_status tree_attn_verify(const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *cu_nodes, const int32_t *kv_start, const int32_t *prefix_len,
                           const uint64_t *anc_bits, int32_t batch, int32_t total_nodes,
                           int32_t max_nodes, int32_t max_prefix, int64_t kv_rows, int32_t hq,
                           int32_t hkv, int32_t head_dim, float scale, tv_dtype dtype, void *out,
                           void *workspace, size_t workspace_bytes, int32_t *err, void *stream);

/*
 * Optional inputs of tree_attn_verify_ex (a NULL pointer: none of them).
 *
 * RoPE inside the call (rope_base > 0).  Defines: [TSD] "The Tree Attention
 * Mechanism", part 3 "Tree Positional IDs": node t is rotated at position
 * pos_ids[t] (from tree_mask_build).  The rotation is tree_rope_apply's (same
 * reading, same base): q is rotated as the kernel loads it (q itself is not
 * written), and the tree's K rows are rotated in place in k_cache, bit for bit
 * as tree_rope_apply writes them, so the cache holds rotated keys for the
 * rounds that follow acceptance.  The call then reads q and the tree's K rows
 * unrotated, i.e. as they come out of the projections.  The workspace also
 * holds each node's cosines and sines (4 * head_dim bytes per node).
 *
 * K/V through a token table (req_to_token != NULL).  Defines: [TSD] "KV
 * Cache Rollback" (paged caches drop unaccepted nodes by page-table updates;
 * kv_rollback_token_table keeps such a table).  Key position p of request b
 * (prefix positions 0 .. P_b - 1, then tree node j at P_b + j) is cache row
 * req_to_token[b * table_stride + p]; kv_start is not read and may be NULL.
 * Every request needs P_b + N_b <= table_stride (else BAD_REQUEST, its output
 * rows not written); an entry outside [0, kv_rows) is reported as BAD_SLOT
 * and row 0 is read in its place (that request's output is then meaningless).
 * req_to_token is 4-byte aligned.
 */
typedef struct {
    const int32_t *pos_ids;      /* [T]; read when rope_base > 0 */
    const int32_t *req_to_token; /* [B, table_stride], or NULL: contiguous rows from kv_start */
    int64_t table_stride;        /* >= 1 when req_to_token is set */
    float rope_base;             /* 0: no rotation; else > 0 and finite (the model's rope theta) */
    int32_t reserved[5];         /* must be zero */
} tv_attn_inputs;

/*
 * Plan overrides for tree_attn_verify: tuning and tests only.
 *
 * tree_attn_verify picks its own plan (how many slices of the key axis each
 * query-row tile is cut into for one request; for batches, a device-side
 * planner that gives every CU an equal share of the key axes, or orders fixed
 * slices longest first) from the host sizes alone, so its workspace size is a
 * pure function of them.  The _ex variants below take an explicit
 * override instead; a NULL override, or zero fields, give exactly the plain
 * calls' plan.  They exist so that tuning sweeps and the tests can reach every
 * plan the kernels support; the results are the same attention (each slice
 * count and order computes the same sums, rounded differently).
 *   splits: key-axis slices per row tile, 0 = the library's choice (clamped
 *           to [1, number of 32-key chunks] for bf16, of 64-key chunks for
 *           fp32);
 *   order:  batches only: TV_ORDER_AUTO (the library's choice: BALANCED
 *           when it applies and no splits are given), TV_ORDER_STATIC
 *           (workgroups take tasks in a fixed order), TV_ORDER_PLANNED (a
 *           planner launch orders them longest first, when the plan is small
 *           enough for it) or TV_ORDER_BALANCED (a planner launch gives each
 *           of 256 persistent workgroups an equal share of the batch's key
 *           axes, cut into a few pieces at request boundaries; batches of at
 *           most 1024 requests with at most 8 row tiles per request and KV
 *           head, else the call falls back to the other orders; splits is
 *           then ignored);
 *   waves:  wavefronts per workgroup of the matrix-core kernel (32 query
 *           rows each), 0 = the library's choice, else 4 or 8.
 */
enum { TV_ORDER_AUTO = 0, TV_ORDER_STATIC = 1, TV_ORDER_PLANNED = 2, TV_ORDER_BALANCED = 3 };
typedef struct {
    int32_t splits;
    int32_t order;
    int32_t waves;
    int32_t reserved[5]; /* must be zero */
} tv_attn_plan_override;

/*
 * tree_attn_verify_ex -- tree_attn_verify with the optional inputs above
 * (in, may be NULL) and a plan override (ov, may be NULL).  With
 * in->rope_base > 0 the call writes k_cache (the tree's K rows); otherwise it
 * only reads it.  With both NULL it is tree_attn_verify.  Its workspace is
 * tree_attn_verify_workspace_size_ex(...) with the same in and ov.
 * Host errors as tree_attn_verify's, plus: TV_ERR_SHAPE for nonzero reserved
 * fields, a rope_base that is negative or not finite, or table_stride < 1 with
 * a table; TV_ERR_NULL for a missing pos_ids (rope on), or a missing kv_start
 * without a table; TV_ERR_ALIGN for a req_to_token not 4-byte aligned.
 */
size_t tree_attn_verify_workspace_size_ex(int32_t batch, int32_t total_nodes, int32_t max_nodes,
                                          int32_t max_prefix, int32_t hq, int32_t hkv, int32_t head_dim,
                                          tv_dtype dtype, const tv_attn_inputs *in,
                                          const tv_attn_plan_override *ov);
tv_status tree_attn_verify_ex(const void *q, void *k_cache, const void *v_cache, const int32_t *cu_nodes,
                              const int32_t *kv_start, const int32_t *prefix_len, const uint64_t *anc_bits,
                              int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix,
                              int64_t kv_rows, int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                              tv_dtype dtype, const tv_attn_inputs *in, void *out, void *workspace,
                              size_t workspace_bytes, int32_t *err, const tv_attn_plan_override *ov,
                              void *stream);

/*
 * tree_attn_verify_plan -- the plan tree_attn_verify(_ex) would run for these
 * host sizes (pure host arithmetic; tuning and tests).  Writes info[0..7]:
 *   [0] 1 = matrix-core kernel (bf16), 0 = vector kernel (fp32)
 *   [1] query rows per workgroup tile   [2] row tiles per (request, KV head)
 *       (both 0 for the vector kernel)
 *   [3] key-axis slices                 [4] keys per slice
 *       (both 0 for the balanced order: its pieces vary in length; 1 and 0
 *       for an unsliced vector-kernel call)
 *   [5] 1 = planned (longest-first) task order for a batch, 2 = balanced
 *   [6] chunks copied ahead of use      [7] workspace bytes without
 *       tv_attn_inputs (saturated to INT32_MAX)
 * Returns the same host-side status the call itself would for these sizes.
 */
tv_status tree_attn_verify_plan(int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix,
                                int32_t hq, int32_t hkv, int32_t head_dim, tv_dtype dtype,
                                const tv_attn_plan_override *ov, int32_t *info);

/*
 * tree_attn_verify_noalloc -- tree_attn_verify for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It takes no workspace and calls no
 * allocating routine.  The split partials and the task table live instead in
 * a static device buffer of TV_NOALLOC_SCRATCH_BYTES per GPU, which each GPU
 * the library runs on holds until the process ends; its address on a device
 * is looked up once, the first time the call runs with that device current.
 *
 * Arguments, plan, kernels and results (bit for bit) are those of
 * tree_attn_verify with the same arguments; so are the errors, plus
 * TV_ERR_SCRATCH (before anything is enqueued) when the plan needs more than
 * TV_NOALLOC_SCRATCH_BYTES, i.e. when tree_attn_verify_workspace_size(...)
 * exceeds it.  All calls on one GPU share that GPU's buffer and each call
 * overwrites it (nothing in it needs to start at zero): two calls that may
 * run at the same time on one GPU (streams without ordering between them)
 * race; order them on one stream.
 */
#define TV_NOALLOC_SCRATCH_BYTES (80u << 20) /* 80 MiB per GPU */
tv_status tree_attn_verify_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *cu_nodes, const int32_t *kv_start,
                                   const int32_t *prefix_len, const uint64_t *anc_bits, int32_t batch,
                                   int32_t total_nodes, int32_t max_nodes, int32_t max_prefix,
                                   int64_t kv_rows, int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                                   tv_dtype dtype, void *out, int32_t *err, void *stream);

/*
 * tree_accept_greedy -- temperature-0 acceptance walk.
 *
 * Defines: [TSD] "Verification and Acceptance Algorithms", greedy tree
 * verification: from the root, look among the current node's children for
 * the one whose draft token equals the target's argmax at the current node;
 * on a match append it and move there, otherwise (or at a leaf) stop; the
 * next starting token is the target's argmax at the last node reached.
 * Readings: the root is implicit and its argmax is root_target[b]; among
 * several matching siblings the lowest index wins; a negative draft token
 * (a dead leaf, [DT] Appendix B) never matches; the walk stops after
 * max_depth accepted nodes.
 *
 * In:  parent, draft_tokens, target_tokens [T] int32 (target_tokens[t] = the
 *      target's argmax after node t); root_target [B]; cu_nodes [B+1].
 * Out: accept_len [B] int32 (0..max_depth); accept_idx [B, max_depth] int32,
 *      request-local node indices in path order, -1 after the path;
 *      next_token [B] int32.
 * err: BAD_REQUEST (cu_nodes outside [0, T] or decreasing).
 */
tv_status tree_accept_greedy(const int32_t *parent, const int32_t *draft_tokens,
                             const int32_t *target_tokens, const int32_t *root_target,
                             const int32_t *cu_nodes, int32_t batch, int32_t total_nodes,
                             int32_t max_depth, int32_t *accept_len, int32_t *accept_idx,
                             int32_t *next_token, int32_t *err, void *stream);

/*
 * tree_accept_stochastic -- the accepted path and next token at temperature
 * T > 0 when the draft is stochastic.
 *
 * Defines: [TSD] "Verification and Acceptance Algorithms", section "Exact
 * Sampling Equivalence": a candidate x that the drafter proposed with
 * probability q(x) is accepted with probability min(1, p(x) / q(x)); after a
 * rejection the replacement comes from (p - q)+ normalised, so that the
 * emitted tokens follow the target's distribution exactly.
 * Reading (the pages do not spell out several candidates at one node): at
 * the current node v (first the implicit root) p = softmax(logits_v / T) and
 * q_v is the distribution v's children were drawn from.  The children are
 * tried in ascending index against the residual r (r = p at first): child c
 * with token x is accepted iff u_accept[c] < min(1, r(x) / q_v(x)) (if
 * q_v(x) = 0: iff r(x) > 0); a rejection replaces r by (r - q_v)+ / its sum
 * (kept if that sum is 0).  An accepted child becomes the current node; the
 * walk ends when no child is accepted, v has none, or max_depth nodes are
 * accepted, and the next token is drawn from r by inverse transform with
 * u_final[b] (the smallest index whose cumulative weight exceeds u times the
 * total; if rounding leaves none, the last index with positive weight).
 * Children with a negative draft token (dead leaves) are skipped.  Float64
 * throughout.  The residual after rejections is formed in closed form: with
 * r = (p - c q_v)+ / W (r = p: c = 0, W = 1), the next one is
 * (p - (c + W) q_v)+ over its sum, which is the update above with the
 * normalisations folded in; so every node's tests are decided at once, in
 * parallel, and the walk follows them.  Only rounding differs from a
 * sequential update.
 *
 * In:  parent, draft_tokens [T] (request-local parents, as tree_mask_build);
 *      cu_nodes [B+1]; root_logits [B, vocab] and node_logits [T, vocab]
 *      (fp32 or bf16: row b is the target at request b's root, row t at node
 *      t; each row needs a finite maximum); root_q [B, vocab], node_q
 *      [T, vocab] fp32 draft probabilities at the same places; u_accept [T],
 *      u_final [B] float64 uniforms in [0, 1) (the call is deterministic in
 *      them).  0 < temperature < inf; 1 <= vocab <= TV_MAX_VOCAB;
 *      1 <= max_depth <= TV_MAX_DEPTH; N_b <= TV_MAX_NODES.  u arrays 8-byte
 *      aligned, the rest naturally aligned.
 * Out: accept_len [B], accept_idx [B, max_depth] (request-local, -1 padded),
 *      next_token [B], as tree_accept_greedy.
 * Workspace: tree_accept_stochastic_workspace_size(batch, total_nodes, vocab)
 *      bytes, 256-byte aligned, no contents required: over the B + T rows,
 *      64 bytes per 2048 logits (chunk statistics and six slots of residual
 *      chunk sums) and 332 bytes per row, plus 24 per node and 4 per request.
 * err: BAD_REQUEST (cu_nodes outside [0, T], decreasing, or N_b above
 *      TV_MAX_NODES), BAD_PARENT, BAD_TOKEN (a draft token >= vocab); such a
 *      request gets accept_len 0, no path and next_token -1.  When cu_nodes
 *      decreases, the node ranges of other requests may overlap; their
 *      results are then unspecified (indices stay in range).
 */
size_t tree_accept_stochastic_workspace_size(int32_t batch, int32_t total_nodes, int32_t vocab);
tv_status tree_accept_stochastic(const int32_t *parent, const int32_t *draft_tokens, const int32_t *cu_nodes,
                                 int32_t batch, int32_t total_nodes, int32_t max_depth, const void *root_logits,
                                 const void *node_logits, tv_dtype dtype, float temperature, const float *root_q,
                                 const float *node_q, int32_t vocab, const double *u_accept, const double *u_final,
                                 int32_t *accept_len, int32_t *accept_idx, int32_t *next_token, void *workspace,
                                 size_t workspace_bytes, int32_t *err, void *stream);

/*
 * kv_compact_path -- commit the accepted path's K/V, discard the rest.
 *
 * Defines: [TSD] "KV Cache Rollback": the tree's K/V were appended to the
 * cache for the pass; afterwards the unaccepted nodes are dropped.  Done here
 * as a physical gather so the cache ends up as token-by-token decoding of the
 * accepted path would have left it: for j < L_b = accept_len[b], row
 * kv_start[b] + P_b + j receives (all hkv heads) what row
 * kv_start[b] + P_b + accept_idx[b, j] held before the call.  No other row is
 * written.  Not idempotent: a second call on the same cache gathers again.
 * new_kv_len[b] = P_b + L_b.
 *
 * In/out: k_cache, v_cache [kv_rows, hkv, head_dim] (16-byte aligned).
 * In:  cu_nodes, kv_start, prefix_len, accept_len [B], accept_idx
 *      [B, max_depth] as produced by tree_accept_greedy.
 * Out: new_kv_len [B] int32.
 * err: BAD_REQUEST (sizes as for tree_attn_verify, or L_b outside
 *      [0, min(max_depth, N_b)], as for kv_rollback_token_table: the gather
 *      writes rows P_b .. P_b + L_b - 1, which must lie inside the request);
 *      BAD_PATH (an accept_idx entry outside [0, N_b)).  Such a request is
 *      left untouched.
 */
tv_status kv_compact_path(void *k_cache, void *v_cache, const int32_t *cu_nodes,
                          const int32_t *kv_start, const int32_t *prefix_len,
                          const int32_t *accept_len, const int32_t *accept_idx, int32_t batch,
                          int32_t total_nodes, int32_t max_depth, int64_t kv_rows, int32_t hkv,
                          int32_t head_dim, tv_dtype dtype, int32_t *new_kv_len, int32_t *err,
                          void *stream);

/*
 * tree_accept_commit -- tree_accept_greedy followed by kv_compact_path, in
 * one launch.
 *
 * Defines: the two calls above ([TSD] "Verification and Acceptance
 * Algorithms", greedy tree verification; [TSD] "KV Cache Rollback"), with
 * the same readings; the outputs equal those of tree_accept_greedy then
 * kv_compact_path on the same arguments.  Saves the second launch and the
 * round trip through accept_len / accept_idx between them.
 *
 * In:  parent, draft_tokens, target_tokens [T]; root_target, kv_start,
 *      prefix_len [B]; cu_nodes [B+1].
 * In/out: k_cache, v_cache [kv_rows, hkv, head_dim] (16-byte aligned).
 * Out: accept_len [B]; accept_idx [B, max_depth] (-1 after the path);
 *      next_token [B]; new_kv_len [B] = P_b + accept_len[b].
 * err: BAD_REQUEST (sizes as for tree_attn_verify).  Such a request is left
 *      untouched: none of its outputs and none of its cache rows is written.
 */
tv_status tree_accept_commit(const int32_t *parent, const int32_t *draft_tokens,
                             const int32_t *target_tokens, const int32_t *root_target,
                             const int32_t *cu_nodes, const int32_t *kv_start, const int32_t *prefix_len,
                             int32_t batch, int32_t total_nodes, int32_t max_depth, int64_t kv_rows,
                             int32_t hkv, int32_t head_dim, tv_dtype dtype, void *k_cache, void *v_cache,
                             int32_t *accept_len, int32_t *accept_idx, int32_t *next_token,
                             int32_t *new_kv_len, int32_t *err, void *stream);

/*
 * tree_select_topb -- the draft tree chosen in one step from a frontier ledger.
 *
 * Defines: [DT] section 3.3 and Appendix B.  The drafter records each
 * candidate it scores in a ledger of shape [batch, D, W*k] (path
 * log-probability plus the slot of its parent) and picks the tree in one step
 * once all depths are drafted: the B highest-scoring records of the request,
 * renumbered parents-first with their parent slots translated, and topped up
 * with never-accepted leaves when fewer than B records exist.  [DAR]
 * "2. Deferred Best-First Pruning" adds a per-level bonus beta to every score
 * before the same pick; with beta <= 0 (and W = B) the pick is the tree a
 * sequential best-first heap would grow.
 * Readings: key = score + beta * level (level = t + 1 for ledger depth t),
 * evaluated in double; keys rank descending, equal keys by depth then slot;
 * the output lists the chosen candidates in that rank order; a dead leaf has
 * parent -1 and token -1 (never accepted by tree_accept_greedy).
 *
 * In:  score [B, D, L] float32 (non-finite = empty slot); parent [B, D, L]
 *      int32: -1 at depth 0, else the slot (0..L-1) of the parent candidate
 *      at depth t-1; token [B, D, L] int32.  batch = B >= 0;
 *      1 <= depth <= TV_MAX_DEPTH; lanes = L >= 1 with depth*L <=
 *      TV_MAX_LEDGER; 1 <= budget <= TV_MAX_NODES; beta finite.
 * Out: tree_parent [B, budget] int32 (request-local, parents first),
 *      tree_token [B, budget] int32, n_real [B] int32 = min(budget, finite
 *      slots): positions >= n_real are dead leaves.  The output is the input
 *      of tree_mask_build with cu_nodes[b] = b * budget.
 * err: BAD_LEDGER when a chosen candidate's parent slot is out of range, not
 *      chosen, or ranked after it (only when keys rise along a path, e.g.
 *      beta > 0); that candidate becomes a dead leaf.
 */
tv_status tree_select_topb(const float *score, const int32_t *parent, const int32_t *token,
                           int32_t batch, int32_t depth, int32_t lanes, int32_t budget, float beta,
                           int32_t *tree_parent, int32_t *tree_token, int32_t *n_real, int32_t *err,
                           void *stream);

/*
 * tree_target_argmax -- the target's greedy choice at every node.
 *
 * Defines: [TSD] "Verification and Acceptance Algorithms", greedy tree
 * verification: the target prediction at a node is the argmax of the logits
 * the verification pass produced there; these choices are the
 * target_tokens (and root_target) of tree_accept_greedy.
 * Readings: the lowest index wins a tie (-0 equals +0); a NaN ranks above
 * every number, so a row holding NaN gives its first NaN.
 *
 * In:  logits [rows, vocab] in dtype (fp32 or bf16), row-major.
 *      0 <= rows <= TV_MAX_TOTAL_NODES; 1 <= vocab <= TV_MAX_VOCAB.
 * Out: token [rows] int32.
 * No device-side errors.
 */
tv_status tree_target_argmax(const void *logits, int32_t rows, int32_t vocab, tv_dtype dtype,
                             int32_t *token, void *stream);

/*
 * tree_target_sample -- the target's sampled choice at every node (T > 0).
 *
 * Defines: [DT] section 4.1: at temperature T > 0 the target token at each
 * node is sampled from the target's distribution while the draft stays
 * deterministic; [TSD] "Verification and Acceptance Algorithms", stochastic
 * verification: with such a (point-mass) draft the min(1, p/q) test accepts a
 * child exactly when the target's sample equals its token, so these tokens are
 * the target_tokens (and root_target) of tree_accept_greedy at T > 0.
 * Row r's token is drawn from softmax(logits[r] / temperature) by inverse
 * transform with the caller's uniform u[r]: with y = x / T, M = max y and
 * w_i = exp(y_i - M), the token is the smallest i with
 * w_0 + ... + w_i > u[r] * (w_0 + ... + w_{vocab-1}), all in float64.
 * Readings: if rounding leaves no such i (or u[r] is not in [0, 1)), the last
 * index with w_i > 0; a row holding NaN gives its first NaN, else a row
 * holding +inf its first +inf; a row of -inf gives 0.  The uniforms are an
 * input, so the call is deterministic; the summation order differs from a
 * sequential sum only by rounding.
 *
 * In:  logits [rows, vocab] in dtype (fp32 or bf16), row-major, 16-byte
 *      aligned; u [rows] float64 (8-byte aligned), the caller's uniforms.
 *      0 < temperature < inf.  0 <= rows <= TV_MAX_TOTAL_NODES,
 *      1 <= vocab <= TV_MAX_VOCAB, rows * ceil(vocab / 2048) < 2^31.
 * Out: token [rows] int32.
 * Workspace: caller-owned device memory of at least
 *      tree_target_sample_workspace_size(rows, vocab) bytes (24 bytes per
 *      2048 logits), 8-byte aligned; overwritten, no contents required.
 * Errors (host, before any launch): SHAPE (negative sizes, temperature not in
 *      (0, inf)), LIMIT, DTYPE, NULL, ALIGN, WORKSPACE.  No device-side errors.
 */
size_t tree_target_sample_workspace_size(int32_t rows, int32_t vocab);
tv_status tree_target_sample(const void *logits, int32_t rows, int32_t vocab, tv_dtype dtype,
                             float temperature, const double *u, int32_t *token, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * tree_rope_apply -- rotary position embedding at the tree's position ids.
 *
 * Defines: [TSD] "The Tree Attention Mechanism", part 3 "Tree Positional IDs":
 * the position a node's RoPE sees is PosID(root) + depth, i.e. pos_ids from
 * tree_mask_build, not the node's index in the flattened tree.
 * Reading (the pages name RoPE without its formula): the rotate-half layout,
 * channel i paired with channel i + d/2, rotated by the angle
 * pos * base^(-2i/d) for i < d/2 (base = the model's rope theta, 1e6 for
 * Qwen3).  Angles, sines, cosines and the rotation are computed in double;
 * each element is rounded once to dtype (bf16 through float: within one
 * bf16 ulp of the exact value).
 *
 * In/out: q [T, hq, head_dim] (every node, every query head) and the tree's
 *      K rows of k_cache [kv_rows, hkv, head_dim] (row kv_start[b] + P_b + j
 *      for node j of request b), rotated in place.  Prefix rows are not
 *      touched.  16-byte aligned.
 * In:  pos_ids [T] int32; cu_nodes [B+1]; kv_start, prefix_len [B].
 *      head_dim in {64, 128}; base > 0 and finite.
 * err: BAD_REQUEST (a node outside every request, or a tree row outside the
 *      cache); that row is not rotated.
 */
tv_status tree_rope_apply(void *q, void *k_cache, const int32_t *pos_ids, const int32_t *cu_nodes,
                          const int32_t *kv_start, const int32_t *prefix_len, int32_t batch,
                          int32_t total_nodes, int64_t kv_rows, int32_t hq, int32_t hkv, int32_t head_dim,
                          float base, tv_dtype dtype, int32_t *err, void *stream);

/*
 * kv_rollback_token_table -- discard the unaccepted nodes of a paged cache by
 * updating its token table; no K/V moves.
 *
 * Defines: [TSD] "KV Cache Rollback": unaccepted tree nodes are discarded "by
 * page table updates in PagedAttention systems".
 * Reading: pages of one token (a token table as in token-level KV pools):
 * req_to_token[b * table_stride + p] is the cache slot of position p of
 * request b, and node j of request b was written to slot tree_slots[lo + j]
 * (lo = cu_nodes[b]).  Afterwards positions P_b .. P_b + L_b - 1 hold the
 * accepted nodes' slots in path order; gathering K/V through the table then
 * gives what kv_compact_path leaves in a contiguous cache.
 *
 * In/out: req_to_token [B, table_stride] int32 (only positions
 *      P_b .. P_b + L_b - 1 are written).
 * In:  tree_slots [T]; cu_nodes [B+1]; prefix_len, accept_len [B];
 *      accept_idx [B, max_depth] from tree_accept_greedy.
 * Out: new_len [B] = P_b + L_b; freed_slots [T]: from offset cu_nodes[b],
 *      the slots of request b's unaccepted nodes in node order, then -1 up
 *      to N_b; n_freed [B] = N_b - L_b.
 * err: BAD_REQUEST (cu_nodes outside [0, T] or decreasing, L_b outside
 *      [0, min(max_depth, N_b)], or P_b + L_b > table_stride); BAD_PATH (an
 *      accept_idx entry outside [0, N_b)).  Such a request is untouched.
 */
tv_status kv_rollback_token_table(int32_t *req_to_token, int64_t table_stride, const int32_t *tree_slots,
                                  const int32_t *cu_nodes, const int32_t *prefix_len,
                                  const int32_t *accept_len, const int32_t *accept_idx, int32_t batch,
                                  int32_t total_nodes, int32_t max_depth, int32_t *new_len,
                                  int32_t *freed_slots, int32_t *n_freed, int32_t *err, void *stream);

/*
 * Tree-aware recurrent verification for a Gated-DeltaNet layer: three calls.
 *
 * Defines: [DT] section 4.5.4, "Tree-aware recurrent verification": in a
 * recurrent layer every tree node needs the state of its own root path and a
 * dense convolution window made of its own ancestors, and only the accepted
 * path's recurrent state is committed (a chain recurrence over the flattened
 * tree lets rejected siblings write into the state later nodes read).
 * Readings (the page gives no formulas): the gated delta rule with
 * L2-normalised queries and keys,
 *   k^ = k / sqrt(|k|^2 + 1e-6),  q^ = scale * q / sqrt(|q|^2 + 1e-6)
 *   S_t = exp(g_t) S_p (I - beta_t k^_t k^_t^T) + beta_t v_t k^_t^T,  o_t = S_t q^_t
 * (p = the node's parent; the request's committed state S0 for a root
 * child; with l2norm = 0, k^ = k and q^ = scale * q), value head h reading
 * query/key head h / (hv / hk), S of shape [dv, dk] per value head; and a
 * depthwise causal convolution of width conv_k with SiLU whose window for a
 * node is the committed conv state (the conv_k - 1 most recent inputs, oldest
 * first) followed by the inputs along the node's root path.
 * Element types: the layer's activations (x, conv state, taps, y, q, k, v) are
 * bf16; g, beta, the state and the outputs are float32.  head_dim (dk = dv)
 * must be TV_GDN_HEAD_DIM.
 */

/*
 * tree_gdn_conv -- the short convolution over each node's ancestor window.
 *
 * In:  x [T, channels] bf16 (the layer's mixed q/k/v inputs per node);
 *      conv_state [B, conv_k - 1, channels] bf16; weight [channels, conv_k]
 *      bf16 (weight[c][conv_k - 1] multiplies the node's own input); parent
 *      [T] (request-local, parent[i] < i); cu_nodes [B+1].  conv_k in
 *      {2, 3, 4}; channels a positive multiple of 8; x, conv_state, weight, y
 *      16-byte aligned.
 * Out: y [T, channels] bf16 = SiLU(sum_i weight[c][i] window[i][c]), computed
 *      in float32 and rounded once.
 * err: BAD_REQUEST (a node outside every request); BAD_PARENT (a parent read
 *      on a window outside [-1, i); the walk stops there as at a root).
 */
tv_status tree_gdn_conv(const void *x, const void *conv_state, const void *weight, const int32_t *parent,
                        const int32_t *cu_nodes, int32_t batch, int32_t total_nodes, int32_t channels,
                        int32_t conv_k, void *y, int32_t *err, void *stream);

/*
 * tree_gdn_verify -- every node's Gated-DeltaNet output, each node seeing the
 * recurrence over its own root path only.
 *
 * In:  q [T, hk, 128], k [T, hk, 128], v [T, hv, 128] bf16 with a common row
 *      stride of row_stride elements (q, k and v may be views into the
 *      output of tree_gdn_conv); row_stride a multiple of 8 and q, k, v
 *      16-byte aligned.  g [T, hv] (log decay), beta [T, hv] float32; state
 *      [B, hv, 128, 128] float32 (S0 of each request, row i = value
 *      channel), 16-byte aligned, not modified; parent [T]; cu_nodes [B+1].
 *      1 <= max_depth <= TV_MAX_DEPTH (levels of the deepest node);
 *      hv % hk == 0; scale finite; l2norm 0 or 1.
 * Out: out [T, hv, 128] float32.
 * Limits per request (device-checked): N_b <= TV_GDN_MAX_NODES and
 *      N_b * max_depth <= TV_GDN_MAX_TABLE, else LIMIT.
 * Arithmetic: dot products of bf16 rows on the matrix cores with float32
 *      accumulation; S0 enters those products as a bf16 pair hi + lo (about
 *      16 significant bits); the rest in float32.
 * err: BAD_REQUEST, LIMIT, BAD_PARENT, TOO_DEEP (level > max_depth).
 */
tv_status tree_gdn_verify(const void *q, const void *k, const void *v, int64_t row_stride, const float *g,
                          const float *beta, const float *state, const int32_t *parent, const int32_t *cu_nodes,
                          int32_t batch, int32_t total_nodes, int32_t max_depth, int32_t hk, int32_t hv,
                          int32_t head_dim, float scale, int32_t l2norm, float *out, int32_t *err, void *stream);

/*
 * tree_gdn_commit -- keep only the accepted path's recurrent state.
 *
 * In/out: state [B, hv, 128, 128] float32: S0 advanced by the accepted
 *      tokens in path order, one step at a time in float32; conv_state
 *      [B, conv_k - 1, channels] bf16: the last conv_k - 1 entries of
 *      (old conv state, x of the accepted nodes).  A request with
 *      accept_len 0 is untouched.
 * In:  x [T, channels] bf16 (the inputs tree_gdn_conv read); k, v,
 *      row_stride, g, beta, hk, hv, head_dim, l2norm as in tree_gdn_verify;
 *      cu_nodes [B+1]; accept_len [B], accept_idx [B, max_depth] from
 *      tree_accept_greedy; conv_k, channels as in tree_gdn_conv.
 * err: BAD_REQUEST (L_b outside [0, min(max_depth, N_b)]), BAD_PATH (an
 *      accept_idx entry outside [0, N_b)); such a request is untouched.
 */
tv_status tree_gdn_commit(float *state, void *conv_state, const void *x, const void *k, const void *v,
                          int64_t row_stride, const float *g, const float *beta, const int32_t *cu_nodes,
                          const int32_t *accept_len, const int32_t *accept_idx, int32_t batch, int32_t total_nodes,
                          int32_t max_depth, int32_t hk, int32_t hv, int32_t head_dim, int32_t channels,
                          int32_t conv_k, int32_t l2norm, int32_t *err, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* TREEVERIFY_H */
