// Internal launchers behind the C ABI (capi.hip).  Arguments are already
// validated on the host when these run; each returns the hipError_t of its
// launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "treeverify.h"

namespace tv {

hipError_t launch_mask_build(const int32_t *parent, const int32_t *cu_nodes, const int32_t *prefix_len,
                             int batch, int total_nodes, int max_nodes, int max_depth, uint64_t *anc,
                             int32_t *level, int32_t *pos, int32_t *err, hipStream_t stream);

hipError_t launch_accept_greedy(const int32_t *parent, const int32_t *draft, const int32_t *target,
                                const int32_t *root_target, const int32_t *cu_nodes, int batch,
                                int total_nodes, int max_depth, int32_t *accept_len, int32_t *accept_idx,
                                int32_t *next_token, int32_t *err, hipStream_t stream);

hipError_t launch_accept_commit(const int32_t *parent, const int32_t *draft, const int32_t *target,
                                const int32_t *root_target, const int32_t *cu_nodes,
                                const int32_t *kv_start, const int32_t *prefix_len, int batch,
                                int total_nodes, int max_depth, int64_t kv_rows, int hkv, int head_dim,
                                tv_dtype dtype, void *k, void *v, int32_t *accept_len,
                                int32_t *accept_idx, int32_t *next_token, int32_t *new_len, int32_t *err,
                                hipStream_t stream);
hipError_t launch_kv_compact(void *k, void *v, const int32_t *cu_nodes, const int32_t *kv_start,
                             const int32_t *prefix_len, const int32_t *accept_len,
                             const int32_t *accept_idx, int batch, int total_nodes, int max_depth,
                             int64_t kv_rows, int hkv, int head_dim, tv_dtype dtype, int32_t *new_len,
                             int32_t *err, hipStream_t stream);

hipError_t launch_select_topb(const float *score, const int32_t *parent, const int32_t *token, int batch,
                              int depth, int lanes, int budget, float beta, int32_t *tree_parent,
                              int32_t *tree_token, int32_t *n_real, int32_t *err, hipStream_t stream);

hipError_t launch_target_argmax(const void *logits, int rows, int vocab, tv_dtype dtype, int32_t *token,
                                hipStream_t stream);
size_t target_sample_workspace(int rows, int vocab);
int64_t target_sample_blocks(int rows, int vocab);
hipError_t launch_target_sample(const void *logits, int rows, int vocab, tv_dtype dtype, double inv_t,
                                const double *u, int32_t *token, void *workspace, hipStream_t stream);

// tree_accept_stochastic: workspace bytes and the launch (stats, then walk).
size_t accept_stochastic_workspace(int batch, int total_nodes, int vocab);
hipError_t launch_accept_stochastic(const int32_t *parent, const int32_t *draft, const int32_t *cu_nodes, int batch,
                                    int total_nodes, int max_depth, const void *root_logits,
                                    const void *node_logits, tv_dtype dtype, double inv_t, const float *root_q,
                                    const float *node_q, int vocab, const double *u_accept, const double *u_final,
                                    int32_t *accept_len, int32_t *accept_idx, int32_t *next_token, void *workspace,
                                    int32_t *err, hipStream_t stream);

// The tree part of RoPE inside tree_attn_verify: (cos, sin) of every node's
// angles into cs [T, d/2] (float2) and the tree's K rows rotated in place
// (contiguous rows from kv_start, or through the token table when non-null).
hipError_t launch_rope_prep(void *k, const int32_t *pos, const int32_t *cu_nodes, const int32_t *kv_start,
                            const int32_t *prefix_len, const int32_t *table, int64_t table_stride, int batch,
                            int total_nodes, int64_t kv_rows, int hkv, int head_dim, float base, tv_dtype dtype,
                            float2 *cs, int32_t *err, hipStream_t stream);
hipError_t launch_tree_rope(void *q, void *k, const int32_t *pos, const int32_t *cu_nodes, const int32_t *kv_start,
                            const int32_t *prefix_len, int batch, int total_nodes, int64_t kv_rows, int hq, int hkv,
                            int head_dim, float base, tv_dtype dtype, int32_t *err, hipStream_t stream);
hipError_t launch_rollback_table(int32_t *table, int64_t stride, const int32_t *tree_slots, const int32_t *cu_nodes,
                                 const int32_t *prefix_len, const int32_t *accept_len, const int32_t *accept_idx,
                                 int batch, int total_nodes, int max_depth, int32_t *new_len, int32_t *freed,
                                 int32_t *n_freed, int32_t *err, hipStream_t stream);

hipError_t launch_gdn_conv(const void *x, const void *conv_state, const void *weight, const int32_t *parent,
                           const int32_t *cu_nodes, int batch, int total_nodes, int channels, int conv_k, void *y,
                           int32_t *err, hipStream_t stream);
hipError_t launch_gdn_verify(const void *q, const void *k, const void *v, int64_t row_stride, const float *g,
                             const float *beta, const float *state, const int32_t *parent, const int32_t *cu_nodes,
                             int batch, int total_nodes, int max_depth, int hk, int hv, float scale, int l2norm,
                             float *out, int32_t *err, hipStream_t stream);
hipError_t launch_gdn_commit(float *state, void *conv_state, const void *x, const void *k, const void *v,
                             int64_t row_stride, const float *g, const float *beta, const int32_t *cu_nodes,
                             const int32_t *accept_len, const int32_t *accept_idx, int batch, int total_nodes,
                             int max_depth, int hk, int hv, int channels, int conv_k, int l2norm, int32_t *err,
                             hipStream_t stream);

// Problem description shared by the attention kernels.
struct AttnArgs {
    const void *q, *k, *v;
    const int32_t *cu_nodes, *kv_start, *prefix_len;
    const uint64_t *anc;
    int batch, total_nodes, max_nodes, max_prefix;
    int64_t kv_rows;
    int hq, hkv, head_dim;
    float scale;
    tv_dtype dtype;
    void *out;
    int32_t *err;
    // optional inputs: K/V rows through a token table (null: kv_start + p),
    // and each node's (cos, sin) per channel pair for rotating q (null: off)
    const int32_t *table = nullptr;
    int64_t table_stride = 0;
    const float2 *rope_cs = nullptr;
};

// Plan of the MFMA path (split over the key axis, fp32 partials, combine).
struct MfmaPlan {
    bool use = false;      // MFMA path selected for these sizes
    int waves = 0;         // wavefronts per workgroup (4 or 8)
    int row_blocks = 0;    // 32-row blocks per wave (1 or 2)
    int rows_per_tile = 0; // query rows (node x GQA-head pairs) per workgroup
    int row_tiles = 0;     // per (request, KV head), sized for max_nodes
    int splits = 0;        // key-axis splits per row tile (1 = no combine)
    int keys_per_split = 0;
    bool table = false;     // batches: workgroups take their task from a planned table
    int table_slots = 0;    // workgroups launched on the table path
    size_t table_off = 0;   // byte offset of the table in the workspace
    bool balanced = false;  // batches: equal key-axis shares per workgroup, persistent workgroups
    size_t bal_wg_off = 0, bal_piece_off = 0, bal_group_off = 0;  // byte offsets of its tables
    size_t ws_bytes = 0;
};
// ov may be null (the library's own plan).
MfmaPlan plan_attn_mfma(int batch, int total_nodes, int max_nodes, int max_prefix, int hq, int hkv,
                        int head_dim, tv_dtype dtype, const tv_attn_plan_override *ov);
// Copy look-ahead (chunks) the launch uses for this plan.
int attn_mfma_lookahead(const MfmaPlan &plan);
hipError_t launch_attn_mfma(const AttnArgs &a, const MfmaPlan &plan, void *workspace,
                            hipStream_t stream);

// fp32 path (vector units): one workgroup per tile of nodes x query heads of
// one KV head.  plan_attn_valu fills splits, keys_per_split and ws_bytes of a
// plan that does not use the matrix cores: splits > 1 cuts the key axis into
// slices whose partials the workspace holds (a merge kernel combines them).
void plan_attn_valu(int batch, int total_nodes, int max_nodes, int max_prefix, int hq, int hkv, int head_dim,
                    const tv_attn_plan_override *ov, MfmaPlan *plan);
hipError_t launch_attn_valu(const AttnArgs &a, const MfmaPlan &plan, void *workspace, hipStream_t stream);

}  // namespace tv
