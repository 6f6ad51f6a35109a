// tv_launch.h -- launch entry points of the mask, acceptance and table kernels
// (each returns the launch's hipError_t). Nothing here is part of the C ABI.
#pragma once

#include "tv_internal.h"

namespace tv {

// Compute units of the current device (cached per device; 0 if HIP cannot say).
int device_cu_count();
// hipFuncSetAttribute(kernel, MaxDynamicSharedMemorySize, bytes) once per
// (current device, kernel); later calls return hipSuccess at once.
hipError_t raise_dynamic_lds(const void* kernel, int bytes);

hipError_t launch_mask_bits(const int32_t* parent, const int32_t* cu_nodes, int32_t batch,
                            int32_t total_nodes, int32_t words, uint64_t* bits, int32_t* depth,
                            int32_t* err, hipStream_t stream);
hipError_t launch_mask_anchor(const int32_t* parent, const int32_t* cu_nodes, int32_t batch,
                              int32_t total_nodes, int32_t max_nodes, int32_t* anchor_pos,
                              int32_t* branch_depth, int32_t* depth, int32_t* err,
                              hipStream_t stream);
hipError_t launch_accept(const int32_t* parent, const int32_t* draft_tok, const int32_t* target_tok,
                         const int32_t* cu_nodes, int32_t batch, int32_t total_nodes,
                         int32_t max_nodes, int32_t max_depth, int32_t* accept_len, int32_t* path,
                         int32_t* bonus_tok, hipStream_t stream);

hipError_t launch_dcut_select(const float* conf, const int32_t* tokens, int32_t batch,
                              int32_t draft_len, int32_t budget, int32_t* n_keep,
                              int32_t* cu_nodes, int32_t* parent, int32_t* packed_tokens,
                              hipStream_t stream);

hipError_t launch_e2e_tv(const void* target_logits, const void* draft_logits, int32_t dtype,
                         int32_t num_nodes, int32_t vocab, float temperature,
                         const int32_t* cu_branches, int32_t num_branches, float* alpha,
                         float* prefix_prob, float* expected_len, hipStream_t stream);

hipError_t launch_graft_retrieve(const int32_t* adj, int32_t vocab, int32_t k,
                                 const int32_t* root_tokens, int32_t batch,
                                 const int32_t* tmpl_parent, const int32_t* tmpl_rank,
                                 int32_t tmpl_nodes, int32_t* out_tokens, hipStream_t stream);
// bytes of split partial lists the update needs (0: one workgroup per row)
size_t graft_update_workspace(int32_t num_nodes, int32_t vocab, int32_t k, int32_t dtype,
                              bool vec);
bool graft_update_vec(const void* logits, int32_t dtype, int32_t vocab);
hipError_t launch_graft_update(int32_t* adj, int32_t vocab, int32_t k, const void* logits,
                               int32_t dtype, int32_t num_nodes, const int32_t* node_tokens,
                               void* workspace, hipStream_t stream);

// stochastic tree verification: workspace layout (byte offsets of the
// per-node tables and share partials), a pure function of host scalars
struct SampledLayout {
  size_t node, child, step, part, bonus, total;
  int C, S;  // children kept per node, shares per logits row
};
SampledLayout sampled_layout(int32_t total_nodes, int32_t max_children, int32_t vocab);
hipError_t launch_accept_sampled(const int32_t* parent, const int32_t* draft_tok,
                                 const int32_t* cu_nodes, int32_t batch, int32_t total_nodes,
                                 int32_t max_nodes, int32_t max_children, int32_t max_depth,
                                 const void* target_logits, const void* draft_logits,
                                 int32_t dtype, int32_t vocab, float temperature,
                                 const float* u_accept, const float* u_bonus,
                                 int32_t* accept_len, int32_t* path, int32_t* bonus_tok,
                                 void* workspace, hipStream_t stream);

}  // namespace tv
