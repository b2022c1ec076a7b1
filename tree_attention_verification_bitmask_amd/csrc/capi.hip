// C ABI of libtreeverify: host-side argument checks, then dispatch to the
// kernels.  Every check runs before any HIP runtime call, so a rejected call
// enqueues nothing (and the checks can be exercised on a machine without a
// GPU).  The definitions each call implements are cited in treeverify.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "treeverify.h"
#include "tv_launch.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

tv_status launch_status(hipError_t e) { return e == hipSuccess ? TV_OK : TV_ERR_LAUNCH; }

tv_status check_batch(int32_t batch, int32_t total_nodes) {
    if (batch < 0 || total_nodes < 0) return TV_ERR_SHAPE;
    if (total_nodes > TV_MAX_TOTAL_NODES) return TV_ERR_LIMIT;
    if (batch > 65535) return TV_ERR_LIMIT;
    return TV_OK;
}

tv_status check_attn_sizes(int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix,
                           int32_t hq, int32_t hkv, int32_t head_dim, tv_dtype dtype) {
    tv_status st = check_batch(batch, total_nodes);
    if (st != TV_OK) return st;
    if (max_nodes < 1 || max_prefix < 0 || hq < 1 || hkv < 1) return TV_ERR_SHAPE;
    if (hq % hkv != 0) return TV_ERR_SHAPE;
    if (max_nodes > TV_MAX_NODES) return TV_ERR_LIMIT;
    if (hq > 65535) return TV_ERR_LIMIT;
    if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_DTYPE;
    if (head_dim != 64 && head_dim != 128) return TV_ERR_DTYPE;
    // the key axis of one request must fit int32 arithmetic comfortably
    if ((int64_t)max_prefix + max_nodes > (1ll << 30)) return TV_ERR_LIMIT;
    return TV_OK;
}

tv_status check_gdn_heads(int32_t hk, int32_t hv, int32_t head_dim, int32_t max_depth, int64_t row_stride) {
    if (hk < 1 || hv < 1 || hv % hk != 0 || max_depth < 1 || row_stride < 1) return TV_ERR_SHAPE;
    if (hv > 65535 || max_depth > TV_MAX_DEPTH) return TV_ERR_LIMIT;
    if (head_dim != TV_GDN_HEAD_DIM) return TV_ERR_DTYPE;
    if (row_stride % 8 != 0) return TV_ERR_ALIGN;
    return TV_OK;
}

tv_status check_gdn_conv(int32_t total_or_batch, int32_t channels, int32_t conv_k) {
    if (channels < 8 || channels % 8 != 0) return TV_ERR_SHAPE;
    if (conv_k < 2 || conv_k > 4) return TV_ERR_SHAPE;
    const int64_t groups = (channels / 8 + 255) / 256;
    if ((int64_t)total_or_batch * groups > (1ll << 31) - 1) return TV_ERR_LIMIT;
    return TV_OK;
}

// Host-side checks of an override: every reserved field zero, known order.
bool override_ok(const tv_attn_plan_override *ov) {
    if (!ov) return true;
    for (int i = 0; i < 5; ++i)
        if (ov->reserved[i] != 0) return false;
    return ov->splits >= 0 && ov->order >= TV_ORDER_AUTO && ov->order <= TV_ORDER_BALANCED &&
           (ov->waves == 0 || ov->waves == 4 || ov->waves == 8);
}

// The plan of a call: the matrix-core kernel's (bf16), else the vector
// kernel's key-axis slices (fp32).
tv::MfmaPlan attn_plan(int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix, int32_t hq,
                       int32_t hkv, int32_t head_dim, tv_dtype dtype, const tv_attn_plan_override *ov) {
    tv::MfmaPlan plan =
        tv::plan_attn_mfma(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, dtype, ov);
    if (!plan.use) tv::plan_attn_valu(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, ov, &plan);
    return plan;
}

// The size checks shared by the call and its plan query; fills *plan.
tv_status attn_plan_checked(int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix,
                            int32_t hq, int32_t hkv, int32_t head_dim, tv_dtype dtype,
                            const tv_attn_plan_override *ov, tv::MfmaPlan *plan) {
    tv_status st = check_attn_sizes(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, dtype);
    if (st != TV_OK) return st;
    if (!override_ok(ov)) return TV_ERR_SHAPE;
    *plan = attn_plan(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, dtype, ov);
    // the vector kernel's grid: (nodes x slices, head tiles, requests)
    if (!plan->use && (int64_t)max_nodes * plan->splits > INT32_MAX) return TV_ERR_LIMIT;
    if (plan->use) {
        // workgroup and merge-wave indices are int on the device
        const int64_t groups = (int64_t)batch * hkv * plan->splits;
        const int64_t grid = (groups + 7) / 8 * plan->row_tiles * 8;
        const int64_t merge_waves =
            (int64_t)batch * hkv * plan->row_tiles * (plan->rows_per_tile / 32) * (head_dim / 32) * 4;
        if (grid > INT32_MAX || merge_waves > INT32_MAX) return TV_ERR_LIMIT;
    }
    return TV_OK;
}

// Host checks of the optional inputs (null: none): reserved fields zero,
// rope_base 0 or positive and finite, a table with a positive stride.
bool inputs_ok(const tv_attn_inputs *in) {
    if (!in) return true;
    for (int i = 0; i < 5; ++i)
        if (in->reserved[i] != 0) return false;
    if (!(in->rope_base >= 0.f) || !(in->rope_base < INFINITY)) return false;
    return !in->req_to_token || in->table_stride >= 1;
}
bool rope_on(const tv_attn_inputs *in) { return in && in->rope_base > 0.f; }

// Workspace of the call: the plan's, then with RoPE on the nodes' (cos, sin)
// pairs (8 bytes per channel pair) at the next 256-byte boundary.
size_t attn_ws_bytes(const tv::MfmaPlan &plan, const tv_attn_inputs *in, int32_t total_nodes, int32_t head_dim,
                     size_t *rope_off) {
    const size_t ws = plan.ws_bytes;
    const size_t off = (ws + 255) & ~(size_t)255;
    if (rope_off) *rope_off = off;
    if (rope_on(in) && total_nodes > 0) return off + (size_t)total_nodes * (size_t)(head_dim / 2) * 8;
    return ws;
}

// Every host check of tree_attn_verify(_ex) except the workspace's; fills *plan.
tv_status attn_args_checked(const void *q, const void *k_cache, const void *v_cache, const int32_t *cu_nodes,
                            const int32_t *kv_start, const int32_t *prefix_len, const uint64_t *anc_bits,
                            int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix,
                            int64_t kv_rows, int32_t hq, int32_t hkv, int32_t head_dim, float scale, tv_dtype dtype,
                            const tv_attn_inputs *in, const void *out, const tv_attn_plan_override *ov,
                            tv::MfmaPlan *plan) {
    tv_status st =
        attn_plan_checked(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, dtype, ov, plan);
    if (st != TV_OK) return st;
    if (kv_rows < 0) return TV_ERR_SHAPE;
    if (!(scale > 0.f) || scale != scale) return TV_ERR_SHAPE;
    if (!inputs_ok(in)) return TV_ERR_SHAPE;
    const bool paged = in && in->req_to_token;
    if (!cu_nodes || !prefix_len || (!paged && !kv_start)) return TV_ERR_NULL;
    if (total_nodes > 0 && (!q || !out || !anc_bits)) return TV_ERR_NULL;
    if (total_nodes > 0 && rope_on(in) && !in->pos_ids) return TV_ERR_NULL;
    if (kv_rows > 0 && (!k_cache || !v_cache)) return TV_ERR_NULL;
    // a table entry that is out of range is replaced by row 0, which must exist
    if (paged && total_nodes > 0 && kv_rows < 1) return TV_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
        !aligned(anc_bits, 8) || (paged && !aligned(in->req_to_token, 4)))
        return TV_ERR_ALIGN;
    return TV_OK;
}

// Enqueues the call whose arguments have passed the checks above: with RoPE
// on, first the pre-pass (the nodes' (cos, sin) into the workspace at
// rope_off, the tree's K rows rotated in place), then the attention.
tv_status attn_launch(const void *q, void *k_cache, const void *v_cache, const int32_t *cu_nodes,
                      const int32_t *kv_start, const int32_t *prefix_len, const uint64_t *anc_bits, int32_t batch,
                      int32_t total_nodes, int32_t max_nodes, int32_t max_prefix, int64_t kv_rows, int32_t hq,
                      int32_t hkv, int32_t head_dim, float scale, tv_dtype dtype, const tv_attn_inputs *in,
                      void *out, void *workspace, size_t rope_off, int32_t *err, const tv::MfmaPlan &plan,
                      void *stream) {
    if (batch == 0 || total_nodes == 0) return TV_OK;
    tv::AttnArgs a;
    if (in && in->req_to_token) {
        a.table = in->req_to_token;
        a.table_stride = in->table_stride;
    }
    if (rope_on(in)) {
        float2 *cs = (float2 *)((char *)workspace + rope_off);
        const hipError_t e =
            tv::launch_rope_prep(k_cache, in->pos_ids, cu_nodes, kv_start, prefix_len, a.table, a.table_stride,
                                 batch, total_nodes, kv_rows, hkv, head_dim, in->rope_base, dtype, cs, err,
                                 (hipStream_t)stream);
        if (e != hipSuccess) return TV_ERR_LAUNCH;
        a.rope_cs = cs;
    }
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.cu_nodes = cu_nodes;
    a.kv_start = kv_start;
    a.prefix_len = prefix_len;
    a.anc = anc_bits;
    a.batch = batch;
    a.total_nodes = total_nodes;
    a.max_nodes = max_nodes;
    a.max_prefix = max_prefix;
    a.kv_rows = kv_rows;
    a.hq = hq;
    a.hkv = hkv;
    a.head_dim = head_dim;
    a.scale = scale;
    a.dtype = dtype;
    a.out = out;
    a.err = err;
    if (plan.use) return launch_status(tv::launch_attn_mfma(a, plan, workspace, (hipStream_t)stream));
    return launch_status(tv::launch_attn_valu(a, plan, workspace, (hipStream_t)stream));
}

// Scratch of tree_attn_verify_noalloc: one copy per GPU, for the whole
// process.  In host code `scratch` names a host-side stand-in, not device
// memory; the device address of each GPU's copy is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[TV_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on first use.
hipError_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

const char *tv_status_string(int status) {
    switch (status) {
        case TV_OK: return "TV_OK";
        case TV_ERR_NULL: return "TV_ERR_NULL: a required pointer is NULL";
        case TV_ERR_SHAPE: return "TV_ERR_SHAPE: inconsistent or negative sizes";
        case TV_ERR_DTYPE: return "TV_ERR_DTYPE: unsupported dtype or head_dim";
        case TV_ERR_LIMIT: return "TV_ERR_LIMIT: a size exceeds a library limit";
        case TV_ERR_WORKSPACE: return "TV_ERR_WORKSPACE: workspace too small or misaligned";
        case TV_ERR_LAUNCH: return "TV_ERR_LAUNCH: the HIP runtime refused a launch";
        case TV_ERR_ALIGN: return "TV_ERR_ALIGN: a pointer breaks the required alignment";
        case TV_ERR_SCRATCH:
            return "TV_ERR_SCRATCH: the call needs more than the static scratch buffer "
                   "(TV_NOALLOC_SCRATCH_BYTES) of tree_attn_verify_noalloc holds";
        default: return "unknown tv_status";
    }
}

int tv_abi_version(void) { return 1; }

tv_status tree_mask_build(const int32_t *parent, const int32_t *cu_nodes, const int32_t *prefix_len,
                          int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_depth,
                          uint64_t *anc_bits, int32_t *level, int32_t *pos_ids, int32_t *err,
                          void *stream) {
    tv_status st = check_batch(batch, total_nodes);
    if (st != TV_OK) return st;
    if (max_nodes < 1 || max_depth < 1) return TV_ERR_SHAPE;
    if (max_nodes > TV_MAX_NODES || max_depth > TV_MAX_DEPTH) return TV_ERR_LIMIT;
    if (!cu_nodes || !prefix_len) return TV_ERR_NULL;
    if (total_nodes > 0 && (!parent || !anc_bits || !level || !pos_ids)) return TV_ERR_NULL;
    if (!aligned(anc_bits, 8)) return TV_ERR_ALIGN;
    if (batch == 0 || total_nodes == 0) return TV_OK;
    return launch_status(tv::launch_mask_build(parent, cu_nodes, prefix_len, batch, total_nodes,
                                               max_nodes, max_depth, anc_bits, level, pos_ids, err,
                                               (hipStream_t)stream));
}

size_t tree_attn_verify_workspace_size_ex(int32_t batch, int32_t total_nodes, int32_t max_nodes,
                                          int32_t max_prefix, int32_t hq, int32_t hkv, int32_t head_dim,
                                          tv_dtype dtype, const tv_attn_inputs *in,
                                          const tv_attn_plan_override *ov) {
    if (check_attn_sizes(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, dtype) != TV_OK)
        return 0;
    if (!override_ok(ov) || !inputs_ok(in)) return 0;
    const tv::MfmaPlan plan =
        attn_plan(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, dtype, ov);
    return attn_ws_bytes(plan, in, total_nodes, head_dim, nullptr);
}

size_t tree_attn_verify_workspace_size(int32_t batch, int32_t total_nodes, int32_t max_nodes,
                                       int32_t max_prefix, int32_t hq, int32_t hkv, int32_t head_dim,
                                       tv_dtype dtype) {
    return tree_attn_verify_workspace_size_ex(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim,
                                              dtype, nullptr, nullptr);
}

tv_status tree_attn_verify_plan(int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix,
                                int32_t hq, int32_t hkv, int32_t head_dim, tv_dtype dtype,
                                const tv_attn_plan_override *ov, int32_t *info) {
    if (!info) return TV_ERR_NULL;
    tv::MfmaPlan plan;
    const tv_status st =
        attn_plan_checked(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, dtype, ov, &plan);
    if (st != TV_OK) return st;
    info[0] = plan.use ? 1 : 0;
    info[1] = plan.use ? plan.rows_per_tile : 0;
    info[2] = plan.use ? plan.row_tiles : 0;
    info[3] = plan.splits;
    info[4] = plan.keys_per_split;
    info[5] = plan.use ? (plan.balanced ? 2 : plan.table ? 1 : 0) : 0;
    info[6] = plan.use ? tv::attn_mfma_lookahead(plan) : 0;
    info[7] = (int32_t)(plan.ws_bytes > (size_t)INT32_MAX ? INT32_MAX : plan.ws_bytes);
    return TV_OK;
}

tv_status tree_attn_verify_ex(const void *q, void *k_cache, const void *v_cache, const int32_t *cu_nodes,
                              const int32_t *kv_start, const int32_t *prefix_len, const uint64_t *anc_bits,
                              int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix,
                              int64_t kv_rows, int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                              tv_dtype dtype, const tv_attn_inputs *in, void *out, void *workspace,
                              size_t workspace_bytes, int32_t *err, const tv_attn_plan_override *ov,
                              void *stream) {
    tv::MfmaPlan plan;
    const tv_status st = attn_args_checked(q, k_cache, v_cache, cu_nodes, kv_start, prefix_len, anc_bits, batch,
                                           total_nodes, max_nodes, max_prefix, kv_rows, hq, hkv, head_dim, scale,
                                           dtype, in, out, ov, &plan);
    if (st != TV_OK) return st;
    size_t rope_off = 0;
    const size_t need = attn_ws_bytes(plan, in, total_nodes, head_dim, &rope_off);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return TV_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return TV_ERR_ALIGN;
    }
    return attn_launch(q, k_cache, v_cache, cu_nodes, kv_start, prefix_len, anc_bits, batch, total_nodes, max_nodes,
                       max_prefix, kv_rows, hq, hkv, head_dim, scale, dtype, in, out, workspace, rope_off, err,
                       plan, stream);
}

tv_status tree_attn_verify_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *cu_nodes, const int32_t *kv_start,
                                   const int32_t *prefix_len, const uint64_t *anc_bits, int32_t batch,
                                   int32_t total_nodes, int32_t max_nodes, int32_t max_prefix,
                                   int64_t kv_rows, int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                                   tv_dtype dtype, void *out, int32_t *err, void *stream) {
    // Every host check first (nothing touches the runtime before they pass),
    // then the plan's workspace against the buffer's size.
    tv::MfmaPlan plan;
    const tv_status st = attn_args_checked(q, k_cache, v_cache, cu_nodes, kv_start, prefix_len, anc_bits, batch,
                                           total_nodes, max_nodes, max_prefix, kv_rows, hq, hkv, head_dim, scale,
                                           dtype, nullptr, out, nullptr, &plan);
    if (st != TV_OK) return st;
    if (plan.ws_bytes > (size_t)TV_NOALLOC_SCRATCH_BYTES) return TV_ERR_SCRATCH;
    if (batch == 0 || total_nodes == 0) return TV_OK;
    // The current device's buffer (looked up once per device) when the plan
    // needs a workspace at all.
    void *ws = nullptr;
    if (plan.ws_bytes > 0 && scratch_address(&ws) != hipSuccess) return TV_ERR_LAUNCH;
    return attn_launch(q, const_cast<void *>(k_cache), v_cache, cu_nodes, kv_start, prefix_len, anc_bits, batch,
                       total_nodes, max_nodes, max_prefix, kv_rows, hq, hkv, head_dim, scale, dtype, nullptr, out, ws,
                       0, err, plan, stream);
}

tv_status tree_attn_verify(const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *cu_nodes, const int32_t *kv_start, const int32_t *prefix_len,
                           const uint64_t *anc_bits, int32_t batch, int32_t total_nodes,
                           int32_t max_nodes, int32_t max_prefix, int64_t kv_rows, int32_t hq,
                           int32_t hkv, int32_t head_dim, float scale, tv_dtype dtype, void *out,
                           void *workspace, size_t workspace_bytes, int32_t *err, void *stream) {
    // (no optional inputs: k_cache is only read)
    return tree_attn_verify_ex(q, const_cast<void *>(k_cache), v_cache, cu_nodes, kv_start, prefix_len, anc_bits,
                               batch, total_nodes, max_nodes, max_prefix, kv_rows, hq, hkv, head_dim, scale, dtype,
                               nullptr, out, workspace, workspace_bytes, err, nullptr, stream);
}

tv_status tree_accept_greedy(const int32_t *parent, const int32_t *draft_tokens,
                             const int32_t *target_tokens, const int32_t *root_target,
                             const int32_t *cu_nodes, int32_t batch, int32_t total_nodes,
                             int32_t max_depth, int32_t *accept_len, int32_t *accept_idx,
                             int32_t *next_token, int32_t *err, void *stream) {
    tv_status st = check_batch(batch, total_nodes);
    if (st != TV_OK) return st;
    if (max_depth < 1) return TV_ERR_SHAPE;
    if (max_depth > TV_MAX_DEPTH) return TV_ERR_LIMIT;
    if (!cu_nodes || !root_target || !accept_len || !accept_idx || !next_token) return TV_ERR_NULL;
    if (total_nodes > 0 && (!parent || !draft_tokens || !target_tokens)) return TV_ERR_NULL;
    if (batch == 0) return TV_OK;
    return launch_status(tv::launch_accept_greedy(parent, draft_tokens, target_tokens, root_target,
                                                  cu_nodes, batch, total_nodes, max_depth, accept_len,
                                                  accept_idx, next_token, err, (hipStream_t)stream));
}

size_t tree_accept_stochastic_workspace_size(int32_t batch, int32_t total_nodes, int32_t vocab) {
    if (check_batch(batch, total_nodes) != TV_OK || vocab < 1 || vocab > TV_MAX_VOCAB) return 0;
    return tv::accept_stochastic_workspace(batch, total_nodes, vocab);
}

tv_status tree_accept_stochastic(const int32_t *parent, const int32_t *draft_tokens, const int32_t *cu_nodes,
                                 int32_t batch, int32_t total_nodes, int32_t max_depth, const void *root_logits,
                                 const void *node_logits, tv_dtype dtype, float temperature, const float *root_q,
                                 const float *node_q, int32_t vocab, const double *u_accept, const double *u_final,
                                 int32_t *accept_len, int32_t *accept_idx, int32_t *next_token, void *workspace,
                                 size_t workspace_bytes, int32_t *err, void *stream) {
    tv_status st = check_batch(batch, total_nodes);
    if (st != TV_OK) return st;
    if (max_depth < 1 || vocab < 1) return TV_ERR_SHAPE;
    if (!(temperature > 0.f) || !(temperature < INFINITY)) return TV_ERR_SHAPE;
    if (max_depth > TV_MAX_DEPTH || vocab > TV_MAX_VOCAB) return TV_ERR_LIMIT;
    if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_DTYPE;
    if (!cu_nodes || !root_logits || !root_q || !u_final || !accept_len || !accept_idx || !next_token)
        return TV_ERR_NULL;
    if (total_nodes > 0 && (!parent || !draft_tokens || !node_logits || !node_q || !u_accept)) return TV_ERR_NULL;
    const size_t es = dtype == TV_F32 ? 4 : 2;
    if (!aligned(root_logits, es) || !aligned(node_logits, es) || !aligned(root_q, 4) || !aligned(node_q, 4) ||
        !aligned(u_accept, 8) || !aligned(u_final, 8))
        return TV_ERR_ALIGN;
    const size_t need = tv::accept_stochastic_workspace(batch, total_nodes, vocab);
    if (batch > 0) {
        if (!workspace || workspace_bytes < need) return TV_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return TV_ERR_ALIGN;
    }
    if (batch == 0) return TV_OK;
    return launch_status(tv::launch_accept_stochastic(
        parent, draft_tokens, cu_nodes, batch, total_nodes, max_depth, root_logits, node_logits, dtype,
        1.0 / (double)temperature, root_q, node_q, vocab, u_accept, u_final, accept_len, accept_idx, next_token,
        workspace, err, (hipStream_t)stream));
}

tv_status kv_compact_path(void *k_cache, void *v_cache, const int32_t *cu_nodes,
                          const int32_t *kv_start, const int32_t *prefix_len,
                          const int32_t *accept_len, const int32_t *accept_idx, int32_t batch,
                          int32_t total_nodes, int32_t max_depth, int64_t kv_rows, int32_t hkv,
                          int32_t head_dim, tv_dtype dtype, int32_t *new_kv_len, int32_t *err,
                          void *stream) {
    tv_status st = check_batch(batch, total_nodes);
    if (st != TV_OK) return st;
    if (max_depth < 1 || hkv < 1 || kv_rows < 0) return TV_ERR_SHAPE;
    if (max_depth > TV_MAX_DEPTH || hkv > 65535) return TV_ERR_LIMIT;
    if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_DTYPE;
    if (head_dim != 64 && head_dim != 128) return TV_ERR_DTYPE;
    if (!cu_nodes || !kv_start || !prefix_len || !accept_len || !accept_idx || !new_kv_len)
        return TV_ERR_NULL;
    if (kv_rows > 0 && (!k_cache || !v_cache)) return TV_ERR_NULL;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16)) return TV_ERR_ALIGN;
    if (batch == 0) return TV_OK;
    return launch_status(tv::launch_kv_compact(k_cache, v_cache, cu_nodes, kv_start, prefix_len,
                                               accept_len, accept_idx, batch, total_nodes, max_depth,
                                               kv_rows, hkv, head_dim, dtype, new_kv_len, err,
                                               (hipStream_t)stream));
}

tv_status tree_accept_commit(const int32_t *parent, const int32_t *draft_tokens,
                             const int32_t *target_tokens, const int32_t *root_target,
                             const int32_t *cu_nodes, const int32_t *kv_start, const int32_t *prefix_len,
                             int32_t batch, int32_t total_nodes, int32_t max_depth, int64_t kv_rows,
                             int32_t hkv, int32_t head_dim, tv_dtype dtype, void *k_cache, void *v_cache,
                             int32_t *accept_len, int32_t *accept_idx, int32_t *next_token,
                             int32_t *new_kv_len, int32_t *err, void *stream) {
    tv_status st = check_batch(batch, total_nodes);
    if (st != TV_OK) return st;
    if (max_depth < 1 || hkv < 1 || kv_rows < 0) return TV_ERR_SHAPE;
    if (max_depth > TV_MAX_DEPTH || hkv > 65535) return TV_ERR_LIMIT;
    if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_DTYPE;
    if (head_dim != 64 && head_dim != 128) return TV_ERR_DTYPE;
    if (!cu_nodes || !root_target || !kv_start || !prefix_len || !accept_len || !accept_idx ||
        !next_token || !new_kv_len)
        return TV_ERR_NULL;
    if (total_nodes > 0 && (!parent || !draft_tokens || !target_tokens)) return TV_ERR_NULL;
    if (kv_rows > 0 && (!k_cache || !v_cache)) return TV_ERR_NULL;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16)) return TV_ERR_ALIGN;
    if (batch == 0) return TV_OK;
    return launch_status(tv::launch_accept_commit(parent, draft_tokens, target_tokens, root_target, cu_nodes,
                                                  kv_start, prefix_len, batch, total_nodes, max_depth,
                                                  kv_rows, hkv, head_dim, dtype, k_cache, v_cache,
                                                  accept_len, accept_idx, next_token, new_kv_len, err,
                                                  (hipStream_t)stream));
}

tv_status tree_select_topb(const float *score, const int32_t *parent, const int32_t *token,
                           int32_t batch, int32_t depth, int32_t lanes, int32_t budget, float beta,
                           int32_t *tree_parent, int32_t *tree_token, int32_t *n_real, int32_t *err,
                           void *stream) {
    if (batch < 0 || depth < 1 || lanes < 1 || budget < 1) return TV_ERR_SHAPE;
    if (batch > 65535 || depth > TV_MAX_DEPTH || budget > TV_MAX_NODES) return TV_ERR_LIMIT;
    if ((int64_t)depth * lanes > TV_MAX_LEDGER) return TV_ERR_LIMIT;
    if (!(beta == beta) || beta > 3.0e38f || beta < -3.0e38f) return TV_ERR_SHAPE;
    if (!tree_parent || !tree_token || !n_real) return TV_ERR_NULL;
    if (batch > 0 && (!score || !parent || !token)) return TV_ERR_NULL;
    if (batch == 0) return TV_OK;
    return launch_status(tv::launch_select_topb(score, parent, token, batch, depth, lanes, budget, beta,
                                                tree_parent, tree_token, n_real, err, (hipStream_t)stream));
}

tv_status tree_target_argmax(const void *logits, int32_t rows, int32_t vocab, tv_dtype dtype,
                             int32_t *token, void *stream) {
    if (rows < 0 || vocab < 1) return TV_ERR_SHAPE;
    if (rows > TV_MAX_TOTAL_NODES || vocab > TV_MAX_VOCAB) return TV_ERR_LIMIT;
    if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_DTYPE;
    if (rows > 0 && (!logits || !token)) return TV_ERR_NULL;
    if (!aligned(logits, 16)) return TV_ERR_ALIGN;
    if (rows == 0) return TV_OK;
    return launch_status(tv::launch_target_argmax(logits, rows, vocab, dtype, token, (hipStream_t)stream));
}

size_t tree_target_sample_workspace_size(int32_t rows, int32_t vocab) {
    if (rows < 0 || vocab < 1) return 0;
    return tv::target_sample_workspace(rows, vocab);
}

tv_status tree_target_sample(const void *logits, int32_t rows, int32_t vocab, tv_dtype dtype, float temperature,
                             const double *u, int32_t *token, void *workspace, size_t workspace_bytes,
                             void *stream) {
    if (rows < 0 || vocab < 1) return TV_ERR_SHAPE;
    if (!(temperature > 0.f) || !(temperature < INFINITY)) return TV_ERR_SHAPE;
    if (rows > TV_MAX_TOTAL_NODES || vocab > TV_MAX_VOCAB) return TV_ERR_LIMIT;
    if (tv::target_sample_blocks(rows, vocab) > INT32_MAX) return TV_ERR_LIMIT;
    if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_DTYPE;
    if (rows > 0 && (!logits || !u || !token || !workspace)) return TV_ERR_NULL;
    if (!aligned(logits, 16) || !aligned(u, 8) || !aligned(workspace, 8)) return TV_ERR_ALIGN;
    if (workspace_bytes < tv::target_sample_workspace(rows, vocab)) return TV_ERR_WORKSPACE;
    if (rows == 0) return TV_OK;
    const double inv_t = 1.0 / (double)temperature;
    return launch_status(tv::launch_target_sample(logits, rows, vocab, dtype, inv_t, u, token, workspace,
                                                  (hipStream_t)stream));
}

tv_status tree_rope_apply(void *q, void *k_cache, const int32_t *pos_ids, const int32_t *cu_nodes,
                          const int32_t *kv_start, const int32_t *prefix_len, int32_t batch,
                          int32_t total_nodes, int64_t kv_rows, int32_t hq, int32_t hkv, int32_t head_dim,
                          float base, tv_dtype dtype, int32_t *err, void *stream) {
    tv_status st = check_batch(batch, total_nodes);
    if (st != TV_OK) return st;
    if (hq < 1 || hkv < 1 || kv_rows < 0) return TV_ERR_SHAPE;
    if (hq > 65535 || hkv > 65535) return TV_ERR_LIMIT;
    if (!(base > 0.f) || base > 3.0e38f) return TV_ERR_SHAPE;
    if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_DTYPE;
    if (head_dim != 64 && head_dim != 128) return TV_ERR_DTYPE;
    if (!cu_nodes || !kv_start || !prefix_len) return TV_ERR_NULL;
    if (total_nodes > 0 && (!q || !k_cache || !pos_ids)) return TV_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k_cache, 16)) return TV_ERR_ALIGN;
    if (batch == 0 || total_nodes == 0) return TV_OK;
    return launch_status(tv::launch_tree_rope(q, k_cache, pos_ids, cu_nodes, kv_start, prefix_len, batch,
                                              total_nodes, kv_rows, hq, hkv, head_dim, base, dtype, err,
                                              (hipStream_t)stream));
}

tv_status kv_rollback_token_table(int32_t *req_to_token, int64_t table_stride, const int32_t *tree_slots,
                                  const int32_t *cu_nodes, const int32_t *prefix_len,
                                  const int32_t *accept_len, const int32_t *accept_idx, int32_t batch,
                                  int32_t total_nodes, int32_t max_depth, int32_t *new_len,
                                  int32_t *freed_slots, int32_t *n_freed, int32_t *err, void *stream) {
    tv_status st = check_batch(batch, total_nodes);
    if (st != TV_OK) return st;
    if (max_depth < 1 || table_stride < 1) return TV_ERR_SHAPE;
    if (max_depth > TV_MAX_DEPTH) return TV_ERR_LIMIT;
    if (!req_to_token || !cu_nodes || !prefix_len || !accept_len || !accept_idx || !new_len || !n_freed)
        return TV_ERR_NULL;
    if (total_nodes > 0 && (!tree_slots || !freed_slots)) return TV_ERR_NULL;
    if (batch == 0) return TV_OK;
    return launch_status(tv::launch_rollback_table(req_to_token, table_stride, tree_slots, cu_nodes, prefix_len,
                                                   accept_len, accept_idx, batch, total_nodes, max_depth, new_len,
                                                   freed_slots, n_freed, err, (hipStream_t)stream));
}

tv_status tree_gdn_conv(const void *x, const void *conv_state, const void *weight, const int32_t *parent,
                        const int32_t *cu_nodes, int32_t batch, int32_t total_nodes, int32_t channels,
                        int32_t conv_k, void *y, int32_t *err, void *stream) {
    tv_status st = check_batch(batch, total_nodes);
    if (st != TV_OK) return st;
    if ((st = check_gdn_conv(total_nodes, channels, conv_k)) != TV_OK) return st;
    if (!cu_nodes) return TV_ERR_NULL;
    if (total_nodes > 0 && (!x || !conv_state || !weight || !parent || !y)) return TV_ERR_NULL;
    if (!aligned(x, 16) || !aligned(conv_state, 16) || !aligned(weight, 16) || !aligned(y, 16))
        return TV_ERR_ALIGN;
    if (batch == 0 || total_nodes == 0) return TV_OK;
    return launch_status(tv::launch_gdn_conv(x, conv_state, weight, parent, cu_nodes, batch, total_nodes, channels,
                                             conv_k, y, err, (hipStream_t)stream));
}

tv_status tree_gdn_verify(const void *q, const void *k, const void *v, int64_t row_stride, const float *g,
                          const float *beta, const float *state, const int32_t *parent, const int32_t *cu_nodes,
                          int32_t batch, int32_t total_nodes, int32_t max_depth, int32_t hk, int32_t hv,
                          int32_t head_dim, float scale, int32_t l2norm, float *out, int32_t *err, void *stream) {
    tv_status st = check_batch(batch, total_nodes);
    if (st != TV_OK) return st;
    if ((st = check_gdn_heads(hk, hv, head_dim, max_depth, row_stride)) != TV_OK) return st;
    if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return TV_ERR_SHAPE;
    if (l2norm != 0 && l2norm != 1) return TV_ERR_SHAPE;
    if (!cu_nodes) return TV_ERR_NULL;
    if (total_nodes > 0 && (!q || !k || !v || !g || !beta || !state || !parent || !out)) return TV_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(state, 16)) return TV_ERR_ALIGN;
    if ((int64_t)batch * hv * (TV_GDN_HEAD_DIM / 32) > (1ll << 31) - 1) return TV_ERR_LIMIT;
    if (batch == 0 || total_nodes == 0) return TV_OK;
    return launch_status(tv::launch_gdn_verify(q, k, v, row_stride, g, beta, state, parent, cu_nodes, batch,
                                               total_nodes, max_depth, hk, hv, scale, l2norm, out, err,
                                               (hipStream_t)stream));
}

tv_status tree_gdn_commit(float *state, void *conv_state, const void *x, const void *k, const void *v,
                          int64_t row_stride, const float *g, const float *beta, const int32_t *cu_nodes,
                          const int32_t *accept_len, const int32_t *accept_idx, int32_t batch, int32_t total_nodes,
                          int32_t max_depth, int32_t hk, int32_t hv, int32_t head_dim, int32_t channels,
                          int32_t conv_k, int32_t l2norm, int32_t *err, void *stream) {
    tv_status st = check_batch(batch, total_nodes);
    if (st != TV_OK) return st;
    if ((st = check_gdn_heads(hk, hv, head_dim, max_depth, row_stride)) != TV_OK) return st;
    if ((st = check_gdn_conv(batch, channels, conv_k)) != TV_OK) return st;
    if (l2norm != 0 && l2norm != 1) return TV_ERR_SHAPE;
    // one launch: batch * hv * (128 / 32) state workgroups + batch * ceil(channels / 2048) conv workgroups
    if ((int64_t)batch * hv * (TV_GDN_HEAD_DIM / 32) + (int64_t)batch * ((channels / 8 + 255) / 256) >
        (1ll << 31) - 1)
        return TV_ERR_LIMIT;
    if (!state || !conv_state || !cu_nodes || !accept_len || !accept_idx) return TV_ERR_NULL;
    if (total_nodes > 0 && (!x || !k || !v || !g || !beta)) return TV_ERR_NULL;
    if (!aligned(state, 16) || !aligned(conv_state, 16) || !aligned(x, 16)) return TV_ERR_ALIGN;
    if (batch == 0) return TV_OK;
    return launch_status(tv::launch_gdn_commit(state, conv_state, x, k, v, row_stride, g, beta, cu_nodes,
                                               accept_len, accept_idx, batch, total_nodes, max_depth, hk, hv,
                                               channels, conv_k, l2norm, err, (hipStream_t)stream));
}

}  // extern "C"
