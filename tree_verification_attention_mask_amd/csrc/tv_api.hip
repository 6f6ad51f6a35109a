// tv_api.hip -- the library's C ABI: host-side argument checks, launch plans,
// kernel launches. Nothing here allocates, frees or synchronises.
#include <algorithm>
#include <mutex>
#include <vector>

#include "tv_launch.h"

using namespace tv;

// Scratch memory of tv_tree_verify_attn_noalloc: the split partials live in
// this file-scope device array instead of a caller workspace. Each device the
// library runs on holds its own copy until the process ends. Host code never
// uses the array's name as an address: its device address is taken once per
// device with hipGetSymbolAddress and kept below.
static __device__ __align__(256) unsigned char scratch[TV_NOALLOC_SCRATCH_BYTES];

namespace {
inline tv_status_t launched(hipError_t e) { return e == hipSuccess ? TV_OK : TV_ERR_HIP; }

std::mutex g_scratch_mu;
std::vector<void*> g_scratch;  // per device: device address of `scratch`, or null

// Device address of this device's copy of `scratch` (looked up on the first
// call on each device, with that device current); null if HIP cannot give it.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((size_t)dev >= g_scratch.size()) g_scratch.resize(dev + 1, nullptr);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}
// the attention plan aims at one workgroup per compute unit of the current
// device; MI355X's 256 when HIP cannot report the count
inline int32_t plan_cus() {
  const int n = device_cu_count();
  return n > 0 ? n : 256;
}
}  // namespace

extern "C" const char* tv_status_string(int32_t s) {
  switch (s) {
    case TV_OK: return "ok";
    case TV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case TV_ERR_UNSUPPORTED: return "unsupported configuration";
    case TV_ERR_WORKSPACE: return "workspace too small";
    case TV_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

extern "C" tv_status_t tv_tree_mask_build(const int32_t* parent, const int32_t* cu_nodes,
                                          int32_t batch, int32_t total_nodes, int32_t max_nodes,
                                          int32_t kind, int32_t words_per_node, uint64_t* bits,
                                          int32_t* anchor_pos, int32_t* branch_depth,
                                          int32_t* depth, int32_t* err, hipStream_t stream) {
  if (!parent || !cu_nodes || !depth || !err) return TV_ERR_INVALID_ARGUMENT;
  if (batch < 1 || total_nodes < 0 || max_nodes < 1) return TV_ERR_INVALID_ARGUMENT;
  if (kind == TV_MASK_BITS) {
    if (!bits) return TV_ERR_INVALID_ARGUMENT;
    if (max_nodes > 64 * TV_MAX_MASK_WORDS || words_per_node > TV_MAX_MASK_WORDS)
      return TV_ERR_UNSUPPORTED;
    if (words_per_node < 1 || (int64_t)words_per_node * 64 < max_nodes) return TV_ERR_INVALID_ARGUMENT;
    return launched(launch_mask_bits(parent, cu_nodes, batch, total_nodes, words_per_node, bits,
                                     depth, err, stream));
  }
  if (kind == TV_MASK_ANCHOR) {
    if (!anchor_pos || !branch_depth) return TV_ERR_INVALID_ARGUMENT;
    return launched(launch_mask_anchor(parent, cu_nodes, batch, total_nodes, max_nodes,
                                       anchor_pos, branch_depth, depth, err, stream));
  }
  return TV_ERR_INVALID_ARGUMENT;
}

extern "C" size_t tv_tree_verify_attn_workspace_size(int32_t batch, int32_t total_nodes,
                                                     int32_t max_nodes, int32_t max_prefix_len,
                                                     int32_t num_q_heads, int32_t num_kv_heads,
                                                     int32_t head_dim, int32_t dtype) {
  if (batch < 1 || total_nodes < 1 || max_nodes < 1 || max_prefix_len < 0 || num_q_heads < 1 ||
      num_kv_heads < 1)
    return 0;
  return plan_attn(batch, total_nodes, max_nodes, max_prefix_len, num_q_heads, num_kv_heads,
                   head_dim, dtype, plan_cus()).workspace;
}

extern "C" tv_status_t tv_tree_verify_attn_plan(int32_t batch, int32_t total_nodes,
                                                int32_t max_nodes, int32_t max_prefix_len,
                                                int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t dtype, int32_t num_cus,
                                                tv_attn_plan_t* plan) {
  if (!plan) return TV_ERR_INVALID_ARGUMENT;
  if (batch < 1 || total_nodes < 1 || max_nodes < 1 || max_prefix_len < 0 || num_q_heads < 1 ||
      num_kv_heads < 1 || num_q_heads % num_kv_heads || num_cus < 0)
    return TV_ERR_INVALID_ARGUMENT;
  if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return TV_ERR_UNSUPPORTED;
  const AttnPlan p = plan_attn(batch, total_nodes, max_nodes, max_prefix_len, num_q_heads,
                               num_kv_heads, head_dim, dtype, num_cus > 0 ? num_cus : plan_cus());
  plan->num_cus = p.num_cus;
  plan->rows_per_block = dtype == TV_F32 ? 16 : 16 * p.waves * p.rw;
  plan->row_blocks = p.row_blocks;
  plan->splits = p.splits;
  plan->keys_per_split = p.keys_per_split;
  plan->workspace_bytes = p.workspace;
  return TV_OK;
}

namespace {

// Host-side checks of an attention call and its launch plan (shared by the
// workspace and the scratch-array entry points). On TV_OK, `args` and `plan`
// are filled in; the workspace itself is checked by the caller.
tv_status_t prepare_attn(const void* q, const void* k_cache, const void* v_cache,
                         int32_t num_pages, const int32_t* block_table, int32_t max_pages_per_req,
                         const int32_t* prefix_len, const int32_t* cu_nodes, int32_t batch,
                         int32_t total_nodes, int32_t max_nodes, int32_t max_prefix_len,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t page_size, int32_t dtype, float softmax_scale,
                         const tv_mask_t* mask, void* out, float* lse, AttnArgs& a,
                         AttnPlan& plan) {
  if (!q || !k_cache || !v_cache || !block_table || !prefix_len || !cu_nodes || !mask || !out)
    return TV_ERR_INVALID_ARGUMENT;
  if (batch < 1 || total_nodes < 1 || max_nodes < 1 || max_prefix_len < 0 || num_pages < 1 ||
      max_pages_per_req < 1 || num_q_heads < 1 || num_kv_heads < 1 || page_size < 1)
    return TV_ERR_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads) return TV_ERR_INVALID_ARGUMENT;
  if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_INVALID_ARGUMENT;
  if (!(softmax_scale > 0.f) || !(softmax_scale < 3.0e38f)) return TV_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return TV_ERR_UNSUPPORTED;
  if (page_size < 16 || (page_size & (page_size - 1))) return TV_ERR_UNSUPPORTED;
  // 32-bit index arithmetic inside the kernels
  if ((int64_t)num_pages * num_kv_heads * page_size >= (int64_t(1) << 31) ||
      (int64_t)total_nodes * num_q_heads >= (int64_t(1) << 31) ||
      (int64_t)batch * max_pages_per_req >= (int64_t(1) << 31))
    return TV_ERR_UNSUPPORTED;
  MaskDev md{mask->kind, mask->words_per_node, mask->bits, mask->anchor_pos, mask->branch_depth};
  if (md.kind == TV_MASK_BITS) {
    if (!md.bits || md.words < 1) return TV_ERR_INVALID_ARGUMENT;
    if ((int64_t)md.words * 64 < max_nodes) return TV_ERR_INVALID_ARGUMENT;
  } else if (md.kind == TV_MASK_ANCHOR) {
    if (!md.anchor_pos || !md.branch_depth) return TV_ERR_INVALID_ARGUMENT;
  } else {
    return TV_ERR_INVALID_ARGUMENT;
  }
  plan = plan_attn(batch, total_nodes, max_nodes, max_prefix_len, num_q_heads, num_kv_heads,
                   head_dim, dtype, plan_cus());
  if (((int64_t)batch * num_kv_heads * plan.row_blocks + 7) * plan.splits >= (int64_t(1) << 31))
    return TV_ERR_UNSUPPORTED;
  a = AttnArgs{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.max_pages = max_pages_per_req;
  a.prefix_len = prefix_len;
  a.cu_nodes = cu_nodes;
  a.batch = batch;
  a.total_nodes = total_nodes;
  a.max_nodes = max_nodes;
  a.max_prefix_len = max_prefix_len;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.page_size = page_size;
  a.dtype = dtype;
  a.scale = softmax_scale;
  a.mask = md;
  a.out = out;
  a.lse = lse;
  return TV_OK;
}

}  // namespace

extern "C" tv_status_t tv_tree_verify_attn(
    const void* q, const void* k_cache, const void* v_cache, int32_t num_pages,
    const int32_t* block_table, int32_t max_pages_per_req, const int32_t* prefix_len,
    const int32_t* cu_nodes, int32_t batch, int32_t total_nodes, int32_t max_nodes,
    int32_t max_prefix_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t page_size, int32_t dtype, float softmax_scale, const tv_mask_t* mask, void* out,
    float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  AttnArgs a;
  AttnPlan plan;
  const tv_status_t st = prepare_attn(q, k_cache, v_cache, num_pages, block_table,
                                      max_pages_per_req, prefix_len, cu_nodes, batch, total_nodes,
                                      max_nodes, max_prefix_len, num_q_heads, num_kv_heads,
                                      head_dim, page_size, dtype, softmax_scale, mask, out, lse, a,
                                      plan);
  if (st != TV_OK) return st;
  if (plan.workspace > 0) {
    if (!workspace || workspace_bytes < plan.workspace) return TV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return TV_ERR_INVALID_ARGUMENT;
  }
  a.workspace = workspace;
  return launched(launch_attn(a, plan, stream));
}

extern "C" tv_status_t tv_tree_verify_attn_noalloc(
    const void* q, const void* k_cache, const void* v_cache, int32_t num_pages,
    const int32_t* block_table, int32_t max_pages_per_req, const int32_t* prefix_len,
    const int32_t* cu_nodes, int32_t batch, int32_t total_nodes, int32_t max_nodes,
    int32_t max_prefix_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t page_size, int32_t dtype, float softmax_scale, const tv_mask_t* mask, void* out,
    float* lse, hipStream_t stream) {
  AttnArgs a;
  AttnPlan plan;
  const tv_status_t st = prepare_attn(q, k_cache, v_cache, num_pages, block_table,
                                      max_pages_per_req, prefix_len, cu_nodes, batch, total_nodes,
                                      max_nodes, max_prefix_len, num_q_heads, num_kv_heads,
                                      head_dim, page_size, dtype, softmax_scale, mask, out, lse, a,
                                      plan);
  if (st != TV_OK) return st;
  if (plan.workspace > (size_t)TV_NOALLOC_SCRATCH_BYTES) return TV_ERR_WORKSPACE;
  a.workspace = nullptr;
  if (plan.workspace > 0) {
    a.workspace = scratch_address();
    if (!a.workspace) return TV_ERR_HIP;
  }
  return launched(launch_attn(a, plan, stream));
}

extern "C" tv_status_t tv_tree_accept(const int32_t* parent, const int32_t* draft_tok,
                                      const int32_t* target_tok, const int32_t* cu_nodes,
                                      int32_t batch, int32_t total_nodes, int32_t max_nodes,
                                      int32_t max_depth, int32_t* accept_len, int32_t* path,
                                      int32_t* bonus_tok, hipStream_t stream) {
  if (!parent || !draft_tok || !target_tok || !cu_nodes || !accept_len || !path)
    return TV_ERR_INVALID_ARGUMENT;
  if (batch < 1 || total_nodes < 0 || max_nodes < 1 || max_depth < 0) return TV_ERR_INVALID_ARGUMENT;
  if (max_nodes > TV_MAX_ACCEPT_NODES) return TV_ERR_UNSUPPORTED;
  return launched(launch_accept(parent, draft_tok, target_tok, cu_nodes, batch, total_nodes,
                                max_nodes, max_depth, accept_len, path, bonus_tok, stream));
}

extern "C" tv_status_t tv_dcut_select(const float* conf, const int32_t* tokens, int32_t batch,
                                      int32_t draft_len, int32_t budget, int32_t* n_keep,
                                      int32_t* cu_nodes, int32_t* parent, int32_t* packed_tokens,
                                      hipStream_t stream) {
  if (!conf || !tokens || !n_keep || !cu_nodes || !parent || !packed_tokens)
    return TV_ERR_INVALID_ARGUMENT;
  if (batch < 1 || draft_len < 1) return TV_ERR_INVALID_ARGUMENT;
  if ((int64_t)batch * draft_len > TV_MAX_DCUT_DRAFT_POSITIONS) return TV_ERR_UNSUPPORTED;
  if (budget < batch || budget > batch * (draft_len + 1)) return TV_ERR_INVALID_ARGUMENT;
  return launched(launch_dcut_select(conf, tokens, batch, draft_len, budget, n_keep, cu_nodes,
                                     parent, packed_tokens, stream));
}

extern "C" tv_status_t tv_e2e_tv_stats(const void* target_logits, const void* draft_logits,
                                       int32_t dtype, int32_t num_nodes, int32_t vocab,
                                       float temperature, const int32_t* cu_branches,
                                       int32_t num_branches, float* alpha, float* prefix_prob,
                                       float* expected_len, hipStream_t stream) {
  if (!target_logits || !draft_logits || !alpha) return TV_ERR_INVALID_ARGUMENT;
  if (num_nodes < 1 || vocab < 1 || num_branches < 0) return TV_ERR_INVALID_ARGUMENT;
  if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_INVALID_ARGUMENT;
  if (!(temperature > 0.f) || !(temperature < 3.0e38f)) return TV_ERR_INVALID_ARGUMENT;
  if (num_branches > 0 && (!cu_branches || !prefix_prob || !expected_len))
    return TV_ERR_INVALID_ARGUMENT;
  return launched(launch_e2e_tv(target_logits, draft_logits, dtype, num_nodes, vocab, temperature,
                                cu_branches, num_branches, alpha, prefix_prob, expected_len,
                                stream));
}

extern "C" tv_status_t tv_graft_retrieve(const int32_t* adj, int32_t vocab, int32_t k,
                                         const int32_t* root_tokens, int32_t batch,
                                         const int32_t* tmpl_parent, const int32_t* tmpl_rank,
                                         int32_t tmpl_nodes, int32_t* out_tokens,
                                         hipStream_t stream) {
  if (!adj || !root_tokens || !tmpl_parent || !tmpl_rank || !out_tokens)
    return TV_ERR_INVALID_ARGUMENT;
  if (vocab < 1 || k < 1 || batch < 1 || tmpl_nodes < 1) return TV_ERR_INVALID_ARGUMENT;
  if (k > TV_MAX_GRAFT_K || tmpl_nodes > TV_MAX_GRAFT_TEMPLATE) return TV_ERR_UNSUPPORTED;
  for (int j = 0; j < tmpl_nodes; ++j) {  // host template: topological, ranks in range
    if (tmpl_parent[j] < -1 || tmpl_parent[j] >= j) return TV_ERR_INVALID_ARGUMENT;
    if (tmpl_rank[j] < 0 || tmpl_rank[j] >= k) return TV_ERR_INVALID_ARGUMENT;
  }
  return launched(launch_graft_retrieve(adj, vocab, k, root_tokens, batch, tmpl_parent, tmpl_rank,
                                        tmpl_nodes, out_tokens, stream));
}

extern "C" size_t tv_graft_update_workspace_size(int32_t num_nodes, int32_t vocab, int32_t k,
                                                 int32_t dtype) {
  if (vocab < 1 || k < 1 || num_nodes < 1 || k > vocab || k > TV_MAX_GRAFT_K) return 0;
  if (dtype != TV_F32 && dtype != TV_BF16) return 0;
  // the alignment of the logits picks the 16-byte or the one-value path: size
  // for either
  const size_t a = graft_update_workspace(num_nodes, vocab, k, dtype, false);
  const size_t b = graft_update_workspace(num_nodes, vocab, k, dtype, true);
  return a > b ? a : b;
}

extern "C" tv_status_t tv_graft_update(int32_t* adj, int32_t vocab, int32_t k,
                                       const void* target_logits, int32_t dtype,
                                       int32_t num_nodes, const int32_t* node_tokens,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  if (!adj || !target_logits || !node_tokens) return TV_ERR_INVALID_ARGUMENT;
  if (vocab < 1 || k < 1 || num_nodes < 1 || k > vocab) return TV_ERR_INVALID_ARGUMENT;
  if (vocab > TV_MAX_GRAFT_VOCAB) return TV_ERR_UNSUPPORTED;
  if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_INVALID_ARGUMENT;
  if (k > TV_MAX_GRAFT_K) return TV_ERR_UNSUPPORTED;
  const size_t need = graft_update_workspace(num_nodes, vocab, k, dtype,
                                             graft_update_vec(target_logits, dtype, vocab));
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return TV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return TV_ERR_INVALID_ARGUMENT;
  }
  return launched(launch_graft_update(adj, vocab, k, target_logits, dtype, num_nodes, node_tokens,
                                      workspace, stream));
}

extern "C" size_t tv_tree_accept_sampled_workspace_size(int32_t total_nodes, int32_t max_children,
                                                        int32_t vocab) {
  if (total_nodes <= 0 || max_children < 0 || vocab < 1) return 0;
  return sampled_layout(total_nodes, max_children, vocab).total;
}

extern "C" tv_status_t tv_tree_accept_sampled(
    const int32_t* parent, const int32_t* draft_tok, const int32_t* cu_nodes, int32_t batch,
    int32_t total_nodes, int32_t max_nodes, int32_t max_children, int32_t max_depth,
    const void* target_logits, const void* draft_logits, int32_t dtype, int32_t vocab,
    float temperature, const float* u_accept, const float* u_bonus, int32_t* accept_len,
    int32_t* path, int32_t* bonus_tok, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  if (batch < 0 || total_nodes < 0 || max_nodes < 0 || max_children < 0 || max_depth < 0)
    return TV_ERR_INVALID_ARGUMENT;
  if (batch == 0) return TV_OK;
  if (!parent || !draft_tok || !cu_nodes || !target_logits || !draft_logits || !u_accept ||
      !u_bonus || !accept_len || !path || !bonus_tok)
    return TV_ERR_INVALID_ARGUMENT;
  if (vocab < 1 || !(temperature > 0.f) || !(temperature < 3.0e38f))
    return TV_ERR_INVALID_ARGUMENT;
  if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_INVALID_ARGUMENT;
  if (max_nodes > TV_MAX_ACCEPT_NODES || max_children > TV_MAX_SAMPLED_CHILDREN)
    return TV_ERR_UNSUPPORTED;
  if ((int64_t)total_nodes * vocab > INT64_C(1) << 40) return TV_ERR_UNSUPPORTED;
  const size_t need = total_nodes > 0 ? sampled_layout(total_nodes, max_children, vocab).total : 0;
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return TV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return TV_ERR_INVALID_ARGUMENT;
  }
  return launched(launch_accept_sampled(parent, draft_tok, cu_nodes, batch, total_nodes, max_nodes,
                                        max_children, max_depth, target_logits, draft_logits,
                                        dtype, vocab, temperature, u_accept, u_bonus, accept_len,
                                        path, bonus_tok, workspace, stream));
}
