/*
 * treeverify.h -- C ABI of the MI355X (gfx950) tree-verification library.
 *
 * One speculative-decoding verification step over a flattened candidate tree:
 *   1. tv_tree_mask_build  parent[] -> depth and the ancestor-only tree mask
 *   2. tv_tree_verify_attn one target attention layer: every tree node attends
 *                          the request's KV prefix plus its own root path
 *   3. tv_tree_accept      greedy acceptance: longest accepted root-to-leaf path
 *   3s. tv_tree_accept_sampled  acceptance when sampling (temperature > 0):
 *                          recursive rejection sampling on both models' logits
 * and, ahead of them for batches of chain drafts,
 *   0. tv_dcut_select      D-cut verification budget: rank the batch's draft
 *                          positions and pack each request's kept prefix
 * and, after the verification pass when the caller has both models' logits,
 *   4. tv_e2e_tv_stats     SpecOPD E2E-TV statistics: per-node acceptance
 *                          probability 1 - TV(p, q), per-branch prefix products
 *   5. tv_graft_update     Graft: refresh the successor table from the target's
 *                          next-token logits at the verified nodes
 * and, while building the next tree,
 *   6. tv_graft_retrieve   Graft: fill freed slots by expanding a template from
 *                          the current token through that table
 *
 * Sources (four web pages on candidate-tree speculative decoding):
 *   Graft      arXiv:2605.20104 -- 163.com article "浙江大学、阿里巴巴联手破解AI推理瓶颈"
 *   BlockPilot arXiv:2606.31315 -- zhengruan.com article on dynamic block size
 *   D-cut      paper 2607.14647 -- gist.science summary "D-cut: Adaptive Verification
 *              Depth Pruning for Batched Speculative Decoding"
 *   SpecOPD    arXiv:2611.02846 -- lewlh.github.io blog post on branch-parallel OPD
 *
 * Conventions (all calls):
 *   - Every pointer is a DEVICE pointer unless its comment says (host).
 *   - The caller allocates and owns every buffer, including the workspace.
 *     The library never allocates, frees or synchronises; each call only
 *     enqueues kernels on `stream` and returns. Results are ready when the
 *     stream reaches that point.
 *   - Trees are packed ragged: request b owns flattened nodes
 *     [cu_nodes[b], cu_nodes[b+1]). parent[] holds REQUEST-LOCAL indices in
 *     topological order: the root is local node 0 with parent -1 and every
 *     other node i has 0 <= parent[i] < i.
 *   - Shape scalars that size a launch (batch, total_nodes, max_nodes,
 *     max_prefix_len, max_depth) come from the host, so no call reads device
 *     memory back. They must be >= the true values in the device arrays;
 *     if they are not, results are undefined but no access leaves the
 *     buffers described below.
 *   - Returns TV_OK once the work is enqueued, or an error status before
 *     enqueueing anything (bad arguments) / after a failed launch (TV_ERR_HIP).
 *   - Deterministic: the launch plan depends only on host scalars and every
 *     reduction has a fixed order, so repeated calls give identical bits.
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TV_OK = 0,
  TV_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, inconsistent shape */
  TV_ERR_UNSUPPORTED = 2,      /* valid but outside what the kernels implement */
  TV_ERR_WORKSPACE = 3,        /* workspace_bytes below the call's *_workspace_size() */
  TV_ERR_HIP = 4               /* a HIP launch failed */
} tv_status_t;

typedef enum { TV_F32 = 0, TV_BF16 = 1 } tv_dtype_t;

typedef enum {
  TV_MASK_BITS = 0,   /* ancestor bitmask, words_per_node 64-bit words per node */
  TV_MASK_ANCHOR = 1  /* anchor position + branch depth (trunk plus chain branches) */
} tv_mask_kind_t;

/* Per-node limits. */
#define TV_MAX_MASK_WORDS 16          /* BITS form: up to 1024 nodes per request */
#define TV_MAX_ACCEPT_NODES 8192      /* tv_tree_accept: nodes per request */

/*
 * Tree mask, as tv_tree_verify_attn reads it (a host struct of device pointers).
 * BITS:   bits[node * words_per_node + j / 64] bit (j % 64) set  <=>  local tree
 *         node j is node's ancestor or node itself.
 * ANCHOR: local tree key j is visible to local node i  <=>
 *         j <= anchor_pos[i]  or  i - branch_depth[i] < j <= i.
 * Prefix keys (positions < prefix_len[b]) are visible to every node of the
 * request in both forms; only the tree-to-tree block is masked.
 */
typedef struct {
  int32_t kind;                /* tv_mask_kind_t */
  int32_t words_per_node;      /* BITS only: 1 .. TV_MAX_MASK_WORDS */
  const uint64_t* bits;        /* BITS:   [total_nodes][words_per_node] */
  const int32_t* anchor_pos;   /* ANCHOR: [total_nodes] */
  const int32_t* branch_depth; /* ANCHOR: [total_nodes] */
} tv_mask_t;

/*
 * tv_tree_mask_build -- tree positions and the ancestor-only tree mask.
 *
 * Graft §二 (third gear): the hybrid tree of draft and retrieved nodes is
 * flattened into a sequence and its tree position ids and tree mask are
 * rebuilt before one parallel verification pass. SpecOPD §02 (attention
 * table, full-attention/GQA row): the mask is the topological ancestor
 * relation -- a node sees its own ancestor path and the shared trunk, not its
 * siblings' branches nor later trunk tokens. The position id of node i is
 * prefix_len + depth[i].
 *
 *   parent        [total_nodes]  request-local parent indices (see conventions)
 *   cu_nodes      [batch + 1]    node offsets; cu_nodes[0] = 0
 *   batch         (host) number of requests, >= 1
 *   total_nodes   (host) cu_nodes[batch]
 *   max_nodes     (host) >= every request's node count
 *   kind          TV_MASK_BITS or TV_MASK_ANCHOR
 *   words_per_node BITS: 64-bit words per node, ceil(max_nodes/64) <= value <= 16
 *   bits          BITS:   out [total_nodes][words_per_node]
 *   anchor_pos    ANCHOR: out [total_nodes]  last visible trunk index (node itself on the trunk)
 *   branch_depth  ANCHOR: out [total_nodes]  1-based depth inside its branch, 0 on the trunk.
 *                 The trunk is the longest prefix 0..T-1 with parent[k] = k-1; every later
 *                 node must start a branch (parent < T) or continue the previous node's
 *                 branch (parent = i-1).
 *   depth         out [total_nodes]  number of ancestors (root 0)
 *   err           out [batch]  0 = ok; 1 = malformed parent[] (parent[0] != -1, or a
 *                 parent outside [0, i)) or, BITS, more nodes than words_per_node*64, or,
 *                 ANCHOR with max_nodes <= 8192, a request of more than 8192 nodes;
 *                 2 = ANCHOR form impossible for this tree. A request with err != 0 gets
 *                 an all-zero mask (ANCHOR: anchor_pos -1, branch_depth 0) and depth -1.
 * Unused outputs of the other form may be NULL.
 */
tv_status_t tv_tree_mask_build(const int32_t* parent, const int32_t* cu_nodes, int32_t batch,
                               int32_t total_nodes, int32_t max_nodes, int32_t kind,
                               int32_t words_per_node, uint64_t* bits, int32_t* anchor_pos,
                               int32_t* branch_depth, int32_t* depth, int32_t* err,
                               hipStream_t stream);

/*
 * Workspace bytes tv_tree_verify_attn needs for these host shape scalars
 * (split-KV partial results). 0 means no workspace is needed. The launch plan
 * aims at one workgroup per compute unit of the CURRENT device (256 if HIP
 * cannot report the count), so query with the device current that the call
 * will run on.
 */
size_t tv_tree_verify_attn_workspace_size(int32_t batch, int32_t total_nodes, int32_t max_nodes,
                                          int32_t max_prefix_len, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t dtype);

/*
 * Launch plan of tv_tree_verify_attn (host only, nothing is enqueued): how the
 * rows of one kv head are cut into blocks and its keys into splits, and the
 * workspace the split partials take. A pure function of the host scalars and
 * num_cus, the compute-unit count to plan for (0 = the current device's).
 * Returns TV_ERR_INVALID_ARGUMENT / TV_ERR_UNSUPPORTED like tv_tree_verify_attn
 * for shapes it would reject.
 */
typedef struct {
  int32_t num_cus;         /* compute units planned for */
  int32_t rows_per_block;  /* (node, query head) rows of one kv head per workgroup */
  int32_t row_blocks;      /* row blocks per (request, kv head) */
  int32_t splits;          /* key splits (1: no merge) */
  int32_t keys_per_split;  /* keys per split, a multiple of 64 */
  size_t workspace_bytes;  /* = tv_tree_verify_attn_workspace_size for this num_cus */
} tv_attn_plan_t;
tv_status_t tv_tree_verify_attn_plan(int32_t batch, int32_t total_nodes, int32_t max_nodes,
                                     int32_t max_prefix_len, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                     int32_t num_cus, tv_attn_plan_t* plan);

/*
 * tv_tree_verify_attn -- one target attention layer over the flattened tree.
 *
 * Graft §二 (third gear): one parallel verification pass of the target over
 * the flattened tree under the tree mask. SpecOPD §02 (proposal tree): the
 * target shares the trunk KV cache and scores every branch in one pass under
 * the tree mask. D-cut technical summary §2 (pipeline, packing/verification):
 * the kept positions of every request form a contiguous prefix of its block
 * and the packed batch is verified in one pass.
 *
 * For request b, tree node i (local) and query head h, with G = Hq/Hkv and
 * kv head g = h / G, P = prefix_len[b], n = node count of b:
 *   keys   = positions p in [0, P)  U  {P + j : j visible to i under `mask`}
 *   s_p    = softmax_scale * <q[i,h,:], K[p,g,:]>
 *   out    = sum_p softmax(s)_p V[p,g,:]        lse = ln sum_p exp(s_p)
 * where K/V at logical position p of request b live in page
 * block_table[b*max_pages_per_req + p/page_size], slot p % page_size:
 * K[p,g,:] = k_cache[page][g][slot][:], V[p,g,d] = v_cache[page][g][d][slot].
 * The tree nodes' own K/V are at positions P .. P+n-1 (written by the caller).
 *
 *   q            [total_nodes][num_q_heads][head_dim]            dtype
 *   k_cache      [num_pages][num_kv_heads][page_size][head_dim]  dtype
 *   v_cache      [num_pages][num_kv_heads][head_dim][page_size]  dtype (d-major pages:
 *                the page_size keys of one (kv head, d) are contiguous)
 *   num_pages    (host) pages in the caches; page ids are clamped into range
 *   block_table  [batch][max_pages_per_req]  entries past a request's last page may hold any
 *                value (never used for a key); page ids outside [0, num_pages) are clamped
 *   prefix_len   [batch]
 *   cu_nodes     [batch + 1]
 *   max_prefix_len (host) >= every prefix_len
 *   head_dim     64 or 128;  num_q_heads % num_kv_heads == 0
 *   page_size    a power of two >= 16 (16 in the measured configurations)
 *   dtype        TV_BF16 (MFMA path) or TV_F32 (fp32 VALU path)
 *   softmax_scale > 0 and finite, usually 1/sqrt(head_dim)
 *   mask         (host) struct of device pointers, typically from tv_tree_mask_build
 *                (ANCHOR needs every request in anchor form)
 *   out          [total_nodes][num_q_heads][head_dim]  dtype (round to nearest even)
 *   lse          [total_nodes][num_q_heads] fp32 natural log, or NULL
 *   workspace    >= tv_tree_verify_attn_workspace_size(...) bytes, 256-byte aligned,
 *                or NULL when that size is 0. Contents on entry are ignored.
 * Calls that share a workspace must not overlap in time.
 */
tv_status_t tv_tree_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                                int32_t num_pages, const int32_t* block_table,
                                int32_t max_pages_per_req, const int32_t* prefix_len,
                                const int32_t* cu_nodes, int32_t batch, int32_t total_nodes,
                                int32_t max_nodes, int32_t max_prefix_len, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                int32_t dtype, float softmax_scale, const tv_mask_t* mask,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * tv_tree_verify_attn_noalloc -- tv_tree_verify_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, arguments and
 * checks, minus the workspace. The split partials go to a scratch array of
 * TV_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends (its address is looked up on the first call on each
 * device). The call allocates nothing.
 *   Returns TV_ERR_WORKSPACE when the launch plan's partials
 *   (tv_tree_verify_attn_workspace_size) exceed TV_NOALLOC_SCRATCH_BYTES, and
 *   TV_ERR_HIP if the scratch address cannot be obtained.
 * Every call on one device shares that device's scratch array: calls that
 * overlap in time on one device (different streams, or graphs replayed
 * concurrently) race and give undefined results. Nothing in the array needs
 * to start at any value; it keeps whatever the last call left there.
 */
#define TV_NOALLOC_SCRATCH_BYTES (16u << 20)
tv_status_t tv_tree_verify_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                        int32_t num_pages, const int32_t* block_table,
                                        int32_t max_pages_per_req, const int32_t* prefix_len,
                                        const int32_t* cu_nodes, int32_t batch,
                                        int32_t total_nodes, int32_t max_nodes,
                                        int32_t max_prefix_len, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                        int32_t dtype, float softmax_scale, const tv_mask_t* mask,
                                        void* out, float* lse, hipStream_t stream);

/*
 * tv_tree_accept -- greedy acceptance of the longest matching root path.
 *
 * SpecOPD §01: drafted tokens that agree with the target are accepted, the
 * draft is cut at the first divergence and the rest discarded. Graft
 * introduction: the target checks the whole tree at once and keeps the path
 * that goes furthest; Graft §二 (third gear): draft and retrieved nodes face
 * the same rule. BlockPilot §八: accepted length is the survival length of
 * the prefix.
 *
 * Node i > 0 matches iff draft_tok[i] == target_tok[parent[i]] (target_tok[v]
 * is the target's greedy token after node v). A node is accepted iff all
 * nodes on its root path match; the root is always accepted. best = accepted
 * node of greatest depth, ties to the smallest local index.
 *
 *   parent, draft_tok, target_tok  [total_nodes]
 *   cu_nodes     [batch + 1]
 *   max_nodes    (host) >= every request's node count, <= TV_MAX_ACCEPT_NODES
 *   max_depth    (host) path row length - 1
 *   accept_len   out [batch]  depth of best = accepted non-root nodes
 *   path         out [batch][max_depth + 1]  local node ids root..best, then -1;
 *                entries past max_depth are not written
 *   bonus_tok    out [batch]  target_tok[best] (the target's next token), or NULL
 * A request with no nodes has no root: accept_len 0, path all -1, bonus_tok -1.
 * parent[] must be a valid tree (tv_tree_mask_build reports it); on a malformed
 * tree indices are clamped, results are undefined and nothing is read or
 * written out of bounds.
 */
tv_status_t tv_tree_accept(const int32_t* parent, const int32_t* draft_tok,
                           const int32_t* target_tok, const int32_t* cu_nodes, int32_t batch,
                           int32_t total_nodes, int32_t max_nodes, int32_t max_depth,
                           int32_t* accept_len, int32_t* path, int32_t* bonus_tok,
                           hipStream_t stream);

/*
 * tv_dcut_select -- D-cut verification budget over a batch of chain drafts.
 *
 * D-cut technical summary §2 (cross-request pruning; pipeline: scoring and
 * ranking, packing): each draft position is scored by the product of its
 * block's draft confidences up to it (the chance the block survives to that
 * depth); all positions of the batch are ranked together and the best are
 * verified; since scores only fall along a block, every request keeps a
 * prefix, and the kept positions are packed densely. The budget ratio and the
 * profiled cost model that picks it stay with the caller: the call takes the
 * number of verified positions, budget = rho * batch * (draft_len + 1).
 *
 * Scores: position 0 of request b (its current token) is always verified;
 * s(b,k) = fl(s(b,k-1) * c(b,k)) in fp32 for k = 1..draft_len with s(b,0) = 1
 * and every confidence clamped to [0, 1] (NaN -> 0). The budget - batch
 * remaining slots go to the draft positions of largest score, ties to the
 * smaller b, then the smaller k.
 *
 *   conf          [batch][draft_len] fp32; conf[b][k-1] is the confidence of drafted token k
 *   tokens        [batch][draft_len + 1] int32: position 0 = current token, k = drafted token k
 *   budget        (host) batch <= budget <= batch * (draft_len + 1), else TV_ERR_INVALID_ARGUMENT
 *   n_keep        out [batch]: verified positions of request b, 1 .. draft_len + 1
 *   cu_nodes      out [batch + 1]: exclusive scan of n_keep (cu_nodes[batch] = budget)
 *   parent        out [budget]: the packed chain trees (-1 at each request's position 0,
 *                 k - 1 at position k), in the layout tv_tree_mask_build takes
 *   packed_tokens out [budget]: tokens[b][k] for the kept positions, request by request
 * Limits: draft_len >= 1, batch * draft_len <= TV_MAX_DCUT_DRAFT_POSITIONS
 * (TV_ERR_UNSUPPORTED beyond). One workgroup; deterministic.
 */
#define TV_MAX_DCUT_DRAFT_POSITIONS 32768
tv_status_t tv_dcut_select(const float* conf, const int32_t* tokens, int32_t batch,
                           int32_t draft_len, int32_t budget, int32_t* n_keep, int32_t* cu_nodes,
                           int32_t* parent, int32_t* packed_tokens, hipStream_t stream);

/*
 * tv_e2e_tv_stats -- SpecOPD E2E-TV statistics of a set of branches.
 *
 * SpecOPD §02 stage 4 and §03.2: with exact rejection sampling the drafted
 * token at a node is accepted with probability alpha = sum_v min(p_v, q_v)
 * = 1 - TV(p, q), where p and q are the target's and the draft's next-token
 * distributions at that node; a branch is accepted token by token, so the
 * chance of accepting its first k tokens is the product of their alphas and
 * the expected run of accepted tokens is the sum of those products.
 *
 *   target_logits, draft_logits  [num_nodes][vocab], dtype TV_BF16 or TV_F32;
 *                p = softmax(target / T), q = softmax(draft / T); every row needs
 *                a finite maximum
 *   temperature  (host) T > 0 and finite
 *   cu_branches  [num_branches + 1]: branch b is the chain of nodes [cu[b], cu[b+1])
 *                in acceptance order (clamped into [0, num_nodes])
 *   alpha        out [num_nodes] fp32
 *   prefix_prob  out [num_nodes] fp32: product of alpha over the branch up to the node
 *   expected_len out [num_branches] fp32: sum of the branch's prefix products
 * num_branches may be 0 (then cu_branches, prefix_prob, expected_len may be NULL
 * and only alpha is computed). One workgroup per node streams its two rows twice.
 */
tv_status_t tv_e2e_tv_stats(const void* target_logits, const void* draft_logits, int32_t dtype,
                            int32_t num_nodes, int32_t vocab, float temperature,
                            const int32_t* cu_branches, int32_t num_branches, float* alpha,
                            float* prefix_prob, float* expected_len, hipStream_t stream);

/*
 * tv_graft_retrieve -- Graft retrieval: expand a template from each request's
 * current token through the successor table.
 *
 * Graft §二 (second gear): a table in GPU memory holds, per vocabulary token,
 * its k most likely successors, ranked; the slots freed by pruning are filled
 * by expanding a stage-specific template rooted at the current token, one row
 * lookup per template node. The page gives the slot budgets (52 / 36 / 20)
 * but not the template shapes: the template is the caller's.
 *
 *   adj          [vocab][k] int32: row t = successors of token t, best first; -1 = empty
 *   root_tokens  [batch]: each request's current token
 *   tmpl_parent  (host) [tmpl_nodes]: parent template node (< j), or -1 for the current token
 *   tmpl_rank    (host) [tmpl_nodes]: which successor (0 .. k-1) the node takes
 *   out_tokens   out [batch][tmpl_nodes]: retrieved tokens; -1 where the parent has no
 *                token or the table entry is empty or outside [0, vocab)
 * Limits: 1 <= k <= TV_MAX_GRAFT_K, 1 <= tmpl_nodes <= TV_MAX_GRAFT_TEMPLATE
 * (TV_ERR_UNSUPPORTED beyond); a template that is not in topological order or
 * has a rank outside [0, k) is TV_ERR_INVALID_ARGUMENT.
 */
#define TV_MAX_GRAFT_K 16
#define TV_MAX_GRAFT_TEMPLATE 64
tv_status_t tv_graft_retrieve(const int32_t* adj, int32_t vocab, int32_t k,
                              const int32_t* root_tokens, int32_t batch,
                              const int32_t* tmpl_parent, const int32_t* tmpl_rank,
                              int32_t tmpl_nodes, int32_t* out_tokens, hipStream_t stream);

/*
 * tv_graft_update -- Graft online update of the successor table.
 *
 * Graft §二 (third gear) and §五: after the verification pass, the target's
 * next-token distribution at every verified node (accepted or not) replaces
 * the table row of that node's token with the target's k most likely next
 * tokens. Ranking is by logit (softmax is monotone), ties to the smaller
 * token id, NaN as -inf. When several nodes carry the same token, the later
 * node (larger index) writes the row. Tokens outside [0, vocab) update
 * nothing; other rows are untouched.
 *
 *   adj          in/out [vocab][k] int32
 *   target_logits [num_nodes][vocab], dtype TV_BF16 or TV_F32 (16-byte aligned
 *                rows with vocab a multiple of 8 (bf16) / 4 (fp32) take the
 *                vector path; any other layout works, more slowly)
 *   node_tokens  [num_nodes]: the token at each verified node
 *   workspace    >= tv_graft_update_workspace_size(...) bytes, 256-byte aligned,
 *                or NULL when that size is 0 (one workgroup per row); partial
 *                top-k lists of the row shares. Contents on entry are ignored;
 *                calls that share a workspace must not overlap in time.
 * Limits: 1 <= k <= min(TV_MAX_GRAFT_K, vocab); vocab <= TV_MAX_GRAFT_VOCAB
 * (TV_ERR_UNSUPPORTED beyond). A workspace below the size is TV_ERR_WORKSPACE.
 */
#define TV_MAX_GRAFT_VOCAB (1 << 30)
size_t tv_graft_update_workspace_size(int32_t num_nodes, int32_t vocab, int32_t k,
                                      int32_t dtype);
tv_status_t tv_graft_update(int32_t* adj, int32_t vocab, int32_t k, const void* target_logits,
                            int32_t dtype, int32_t num_nodes, const int32_t* node_tokens,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tv_tree_accept_sampled -- stochastic tree verification (sampling at T > 0).
 *
 * The pages verify at temperature 1 (BlockPilot §五, D-cut §4) and give the
 * one-token rule (SpecOPD §03.2: exact rejection sampling accepts a drafted
 * token with the overlap of the target's and the draft's distributions). The
 * rule for a tree is recursive rejection sampling (Jeon et al. 2024,
 * "Recursive Speculative Decoding"), SpecInfer's multi-step speculative
 * sampling with siblings drawn without replacement, under which the emitted
 * tokens follow the target's distribution whatever the draft was:
 *
 * starting at the root, with p = softmax(target_logits[node] / T) and
 * q = softmax(draft_logits[node] / T) (NaN logits count as -inf), the node's
 * children are tried in local index order. The child with token x is
 * accepted iff u_accept[child] * q(x) < p(x) (probability min(1, p(x)/q(x)));
 * the walk then moves to it. On a rejection p becomes the normalised residual
 * max(0, p - q) (unchanged if that is all zero) and x's mass leaves q, which
 * is renormalised. A child whose token is outside [0, vocab) is passed over.
 * When no child is accepted, the bonus token is the smallest v with
 * sum_{w <= v} p(w) > u_bonus[b] * sum_w p(w) (inverse transform in token
 * order; the last token with mass when rounding leaves none).
 *
 *   parent, draft_tok, cu_nodes  as for tv_tree_accept; draft_tok[i] is the
 *                token node i carries (the root's is not tested)
 *   max_nodes    (host) >= every request's node count, <= TV_MAX_ACCEPT_NODES
 *   max_children (host) >= the most children of any node, <= TV_MAX_SAMPLED_CHILDREN
 *   max_depth    (host) path row length - 1
 *   target_logits, draft_logits [total_nodes][vocab], dtype TV_BF16 or TV_F32:
 *                row i = the next-token logits after node i (the draft's row
 *                is the distribution node i's children were drawn from)
 *   temperature  > 0 and finite
 *   u_accept     [total_nodes] uniforms in [0, 1), one per node (a node's own
 *                test uses its entry); u_bonus [batch] uniforms in [0, 1)
 *   accept_len   out [batch]; path out [batch][max_depth + 1] local ids root..last
 *                accepted node, then -1; bonus_tok out [batch] (-1 when the
 *                request is empty or its distribution has no mass)
 *   workspace    >= tv_tree_accept_sampled_workspace_size(total_nodes, max_children,
 *                vocab) bytes, 256-byte aligned: per-node normalisers, children
 *                and rejection steps, and per-share partial sums. Contents on
 *                entry are ignored; calls sharing it must not overlap.
 * Launches max_children + 2 kernels (every node's rejection chain is prepared
 * for all nodes at once, then one walk per request).
 * Decisions are taken in fp32: a uniform within rounding of its threshold may
 * go either way. On a malformed tree indices are clamped and nothing is read or
 * written out of bounds; results are then undefined.
 */
#define TV_MAX_SAMPLED_CHILDREN 512
size_t tv_tree_accept_sampled_workspace_size(int32_t total_nodes, int32_t max_children,
                                             int32_t vocab);
tv_status_t tv_tree_accept_sampled(const int32_t* parent, const int32_t* draft_tok,
                                   const int32_t* cu_nodes, int32_t batch, int32_t total_nodes,
                                   int32_t max_nodes, int32_t max_children, int32_t max_depth,
                                   const void* target_logits, const void* draft_logits,
                                   int32_t dtype, int32_t vocab, float temperature,
                                   const float* u_accept, const float* u_bonus,
                                   int32_t* accept_len, int32_t* path, int32_t* bonus_tok,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code: status is a tv_status_t value (taken
 * as a plain integer, so that any other value is defined input and gives
 * "unknown status"). */
const char* tv_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* TREEVERIFY_H */
